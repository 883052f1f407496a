"""Seeded generators for the five synthetic workloads of the chunk layer.

Every array is produced on the host from ``numpy.random.default_rng`` so the
oracle and the HIP path see identical bits.  Floating inputs that the GPU
consumes in bf16 are rounded here once (round-to-nearest-even) and returned as
float32 arrays holding exactly representable bf16 values.

Workloads (the shapes the pages' own training runs use, synthetic content):
  * tiny H-Net layer, fp32, 2 x 256 bytes, d=64, piecewise-constant h;
        plus a 32 x 8 coding-rate case for brute force.
  * ByteGen-style byte streams: 32-byte packed order-book events
        (ByteGen report, section 2.3 "data preprocessing" and its Fig. 1),
        ragged 32 x U{32..256} events, batch 16, bf16 activations.
  * two-stage H-Net input: those streams at batch 32 (optionally every sequence 8192 bytes)
        driving a two-stage H-Net hierarchy, d 512 -> 768.
  * ByteFlow coding-rate chunking input: unit-norm rows drawn from a
        mixture of 32 Gaussian clusters with random cluster switches, fp32.
  * full ByteFlow layer input: those rows at d=512 in bf16 with a 1536-wide global stand-in and
        16 bin matrices for the multi-linear upsampling.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# one seeded stream per workload
SEED_HNET_TINY = 20260000
SEED_EVENT_STREAMS = 20260001
SEED_HNET_TWO_STAGE = 20260002
SEED_CODING_RATE_FP32 = 20260003
SEED_BYTEFLOW_LAYER = 20260004

# --------------------------------------------------------------------------
# bf16 helpers (input rounding only)
# --------------------------------------------------------------------------


def bf16_bits(x) -> np.ndarray:
    """Round to bf16 with round-to-nearest-even; return the uint16 bit patterns."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def from_bf16_bits(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """fp32 array whose values are exactly the bf16 rounding of ``x``."""
    return from_bf16_bits(bf16_bits(x))


@dataclass
class Ragged:
    """Packed ragged batch: rows of all sequences back to back plus offsets."""
    offsets: np.ndarray  # int64 [nseq+1]

    @property
    def nseq(self) -> int:
        return len(self.offsets) - 1

    @property
    def total(self) -> int:
        return int(self.offsets[-1])

    def lengths(self) -> np.ndarray:
        return np.diff(self.offsets)


def _offsets(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int64)


def _matmul_rows(x, w, chunk=32768):
    """x @ w in float64, chunked over rows to bound memory."""
    out = np.empty((x.shape[0], w.shape[1]), dtype=np.float64)
    for i in range(0, x.shape[0], chunk):
        out[i:i + chunk] = np.asarray(x[i:i + chunk], dtype=np.float64) @ w
    return out


# --------------------------------------------------------------------------
# tiny piecewise-constant activations
# --------------------------------------------------------------------------


def gen_hnet_tiny(seed: int = SEED_HNET_TINY, nseq: int = 2, T: int = 256, d: int = 64):
    """Piecewise-constant N(0,I) segments (lengths U{3..12}) plus noise of
    variance 0.05; Wq, Wk ~ N(0, 1/d).  q = h Wq and k = h Wk (row vectors)."""
    rng = np.random.default_rng(seed)
    h = np.empty((nseq * T, d))
    for s in range(nseq):
        t = 0
        while t < T:
            L = int(rng.integers(3, 13))
            h[s * T + t: s * T + min(t + L, T)] = rng.standard_normal(d)
            t += L
    h += np.sqrt(0.05) * rng.standard_normal(h.shape)
    wq = rng.standard_normal((d, d)) / np.sqrt(d)
    wk = rng.standard_normal((d, d)) / np.sqrt(d)
    f32 = np.float32
    return dict(h=h.astype(f32), q=(h @ wq).astype(f32), k=(h @ wk).astype(f32),
                offsets=_offsets([T] * nseq), d=d, threshold=0.5, dtype="f32")


def cluster_rows(rng, nseq: int, T: int, d: int, ncl: int = 32, sigma: float = 0.25,
                 switch_p: float = 1.0 / 6.0) -> np.ndarray:
    """[nseq, T, d] float64 unit rows from a mixture of ``ncl`` Gaussian
    clusters.  The label switches at each t >= 1 with probability ``switch_p``
    (a Bernoulli stand-in for Poisson switch times of rate 1/6) to a label
    drawn uniformly; row = normalise(mu_label + sigma * xi)."""
    mu = rng.standard_normal((ncl, d))
    out = np.empty((nseq, T, d))
    for s in range(nseq):
        sw = rng.random(T) < switch_p
        newl = rng.integers(ncl, size=T)
        lab = np.empty(T, dtype=np.int64)
        cur = int(rng.integers(ncl))
        for t in range(T):
            if t > 0 and sw[t]:
                cur = int(newl[t])
            lab[t] = cur
        x = mu[lab] + sigma * rng.standard_normal((T, d))
        out[s] = x / np.linalg.norm(x, axis=1, keepdims=True)
    return out


def gen_coding_rate_tiny(seed: int = SEED_HNET_TINY + 100, T: int = 32, d: int = 8, eps2: float = 0.5):
    rng = np.random.default_rng(seed)
    h = cluster_rows(rng, 1, T, d, ncl=4)[0]
    return dict(h=h.astype(np.float32), T=T, d=d, eps2=eps2)


# --------------------------------------------------------------------------
# 32-byte packed order-book events
# --------------------------------------------------------------------------

EPOCH_NS = 1_730_793_600_000_000_000  # 2024-11-05 08:00 UTC
PARETO_SCALE_NS = 171_000.0           # median gap x_m * 2**(1/1.5) = 0.271 ms


def event_bytes(rng, n_events: int) -> np.ndarray:
    """One stream of ``n_events`` packed 32-byte events, little-endian:
    [0] type (0 add, 1 cancel, 2 modify, 3 trade; probs .45/.40/.10/.05),
    [1..7] 55-bit order id << 1 | side, [8..15] uint64 ns timestamp with
    Pareto(1.5) gaps, [16..23] int64 price (+-1 tick random walk from 1e7),
    [24..27] uint32 qty = max(1, round(LogNormal(ln 5, 1))), [28..31] zero."""
    typ = rng.choice(4, size=n_events, p=[0.45, 0.40, 0.10, 0.05]).astype(np.uint64)
    base = int(rng.integers(1 << 40, 1 << 41))
    ids = np.empty(n_events, dtype=np.uint64)
    side = np.empty(n_events, dtype=np.uint64)
    live_ids, live_side = [], []
    nxt = base
    for i in range(n_events):
        if typ[i] == 0 or not live_ids:
            nxt += int(rng.integers(1, 17))
            live_ids.append(nxt)
            live_side.append(int(rng.integers(2)))
            j = len(live_ids) - 1
        else:
            j = len(live_ids) - 1 - int(rng.integers(min(64, len(live_ids))))
        ids[i] = live_ids[j] & ((1 << 55) - 1)
        side[i] = live_side[j]
    gaps = (1.0 + rng.pareto(1.5, size=n_events)) * PARETO_SCALE_NS
    ts = (EPOCH_NS + int(rng.integers(0, 10**12)) + np.cumsum(np.minimum(gaps, 1e13))).astype(np.uint64)
    price = (10**7 + np.cumsum(rng.choice([-1, 1], size=n_events))).astype(np.int64)
    qty = np.maximum(1, np.rint(rng.lognormal(np.log(5.0), 1.0, size=n_events))).astype(np.uint64)
    qty = np.minimum(qty, 0xFFFFFFFF)
    words = np.zeros((n_events, 4), dtype=np.uint64)
    words[:, 0] = typ | (((ids << np.uint64(1)) | side) << np.uint64(8))
    words[:, 1] = ts
    words[:, 2] = price.view(np.uint64)
    words[:, 3] = qty
    return words.astype("<u8").view(np.uint8).reshape(-1)


def _stream_batch(rng, nseq, min_events, max_events, fixed_events):
    if fixed_events is not None:
        nev = [int(fixed_events)] * nseq
    else:
        nev = [int(x) for x in rng.integers(min_events, max_events + 1, size=nseq)]
    streams = [event_bytes(rng, n) for n in nev]
    return np.concatenate(streams), _offsets([32 * n for n in nev])


def _embed_conv(rng, x_bytes, offsets, d):
    """Random byte embedding (256 x d, N(0,1)) then a depthwise causal conv1d
    with kernel 4 (weights N(0, 1/4), no bias, zero left padding per sequence)."""
    emb = rng.standard_normal((256, d))
    w = rng.standard_normal((4, d)) / 2.0
    e = emb[x_bytes]
    h = w[0] * e
    pos = np.arange(len(x_bytes)) - np.repeat(offsets[:-1], np.diff(offsets))
    for j in range(1, 4):
        sh = np.zeros_like(e)
        sh[j:] = e[:-j]
        sh[pos < j] = 0.0
        h += w[j] * sh
    return h


def gen_event_streams(seed: int = SEED_EVENT_STREAMS, nseq: int = 16, d: int = 512, min_events: int = 32,
           max_events: int = 256, fixed_events=None):
    """ByteGen-style streams -> h = conv(embed(bytes)); q = h Wq, k = h Wk,
    Wq, Wk ~ N(0, 1/d); h, q, k rounded to bf16."""
    rng = np.random.default_rng(seed)
    xb, off = _stream_batch(rng, nseq, min_events, max_events, fixed_events)
    h = _embed_conv(rng, xb, off, d)
    wq = rng.standard_normal((d, d)) / np.sqrt(d)
    wk = rng.standard_normal((d, d)) / np.sqrt(d)
    q = bf16_round(_matmul_rows(h, wq))
    k = bf16_round(_matmul_rows(h, wk))
    # wq, wk rounded to bf16 for a projection computed on the device from the bf16 h
    return dict(bytes=xb, offsets=off, h=bf16_round(h), q=q, k=k, d=d, threshold=0.5, dtype="bf16",
                wq=bf16_round(wq), wk=bf16_round(wk))


def gen_hnet_two_stage(seed: int = SEED_HNET_TWO_STAGE, nseq: int = 32, d_local: int = 512, d_mid: int = 768,
           fixed_T=None, min_events: int = 32, max_events: int = 256):
    """Two-stage hierarchy on the event streams.  ``fixed_T`` (multiple of 32)
    makes every sequence that long (8192 for the headline workload).
    Stage thresholds come from the 0.75 score quantile of each stage."""
    fixed_events = None if fixed_T is None else fixed_T // 32
    base = gen_event_streams(seed, nseq=nseq, d=d_local, min_events=min_events, max_events=max_events,
                  fixed_events=fixed_events)
    rng = np.random.default_rng(seed + 7919)
    base["w_mid"] = rng.standard_normal((d_local, d_mid)) / np.sqrt(d_local)
    base["wq2"] = rng.standard_normal((d_mid, d_mid)) / np.sqrt(d_mid)
    base["wk2"] = rng.standard_normal((d_mid, d_mid)) / np.sqrt(d_mid)
    base["w_back"] = rng.standard_normal((d_mid, d_local)) / np.sqrt(d_mid)
    base.update(d_mid=d_mid, quantile=0.75)
    return base


def gen_stage2_inputs(z1, cfg):
    """Stand-in for the stage-1 main network's input projection: x2 = z1 W_mid,
    q2 = x2 Wq2, k2 = x2 Wk2 (all rounded to bf16)."""
    x2 = bf16_round(_matmul_rows(z1, cfg["w_mid"]))
    return dict(x2=x2, q2=bf16_round(_matmul_rows(x2, cfg["wq2"])),
                k2=bf16_round(_matmul_rows(x2, cfg["wk2"])))


def gen_stage2_backproj(y2, cfg):
    """Stand-in projection of the stage-2 result back to d_local (bf16)."""
    return bf16_round(_matmul_rows(y2, cfg["w_back"]))


# --------------------------------------------------------------------------
# ByteFlow coding-rate inputs
# --------------------------------------------------------------------------


def gen_coding_rate_fp32(seed: int = SEED_CODING_RATE_FP32, nseq: int = 8, T: int = 8192, d: int = 256,
           eps2: float = 0.5, K: int = 2048):
    rng = np.random.default_rng(seed)
    h = cluster_rows(rng, nseq, T, d).astype(np.float32)
    return dict(h=h, nseq=nseq, T=T, d=d, eps2=eps2, K=K, dtype="f32")


def gen_byteflow_layer(seed: int = SEED_BYTEFLOW_LAYER, nseq: int = 32, T: int = 8192, d_local: int = 512,
           d_global: int = 1536, K: int = 2048, nbins: int = 16, eps2: float = 0.5):
    rng = np.random.default_rng(seed)
    h = bf16_round(cluster_rows(rng, nseq, T, d_local))
    w_g = rng.standard_normal((d_local, d_global)) / np.sqrt(d_local)
    w_bin = bf16_round(rng.standard_normal((nbins, d_global, d_local)) / np.sqrt(d_global))
    # routing projections for the cosine-score variant of the chunker (drawn
    # after everything above, so those arrays are unchanged)
    wq = bf16_round(rng.standard_normal((d_local, d_local)) / np.sqrt(d_local))
    wk = bf16_round(rng.standard_normal((d_local, d_local)) / np.sqrt(d_local))
    return dict(h=h, w_g=w_g, w_bin=w_bin, wq=wq, wk=wk, nseq=nseq, T=T, d_local=d_local,
                d_global=d_global, K=K, nbins=nbins, eps2=eps2, dtype="bf16")


def gen_cosine_qk(h, cfg, rows=None):
    """q = h Wq, k = h Wk for the cosine-score chunker (fp64 products of the
    bf16 inputs, rounded to bf16); ``rows`` limits it to h[:rows]."""
    hh = np.asarray(h).reshape(-1, h.shape[-1])
    if rows is not None:
        hh = hh[:rows]
    return bf16_round(_matmul_rows(hh, cfg["wq"])), bf16_round(_matmul_rows(hh, cfg["wk"]))


def gen_global_standin(z, cfg):
    """Stand-in for W_proj followed by the global Transformer: g = z W_g (bf16)."""
    zz = np.asarray(z).reshape(-1, z.shape[-1])
    return bf16_round(_matmul_rows(zz, cfg["w_g"])).reshape(z.shape[:-1] + (cfg["w_g"].shape[1],))
