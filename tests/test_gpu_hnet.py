"""GPU parity: H-Net route / quantile / compact / EMA dechunk against the oracle."""
import numpy as np
import pytest

import oracle
from synthdata import (bf16_round, gen_hnet_tiny, gen_event_streams, gen_hnet_two_stage, gen_stage2_inputs,
                       gen_stage2_backproj)
from tests.helpers import to_dev, to_np, row_rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import byte_level_lm_amd as B
    B.lib()
    return B


def _torch():
    import torch
    return torch


def _ragged(rng, lengths, d, dtype):
    torch = _torch()
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = int(off[-1])
    q = rng.standard_normal((N, d)).astype(np.float32)
    k = rng.standard_normal((N, d)).astype(np.float32)
    h = rng.standard_normal((N, d)).astype(np.float32)
    if dtype == torch.bfloat16:
        from synthdata import bf16_round
        q, k, h = bf16_round(q), bf16_round(k), bf16_round(h)
    return off, q, k, h


def _check_route(ops, q, k, off, dtype, threshold=0.5):
    p, b, tau = ops.route(to_dev(q, dtype), to_dev(k, dtype), to_dev(off), threshold=threshold)
    p_g, b_g = to_np(p), to_np(b).astype(bool)
    p_o = oracle.route(q, k, off)
    assert np.max(np.abs(p_g - p_o)) < 5e-6
    assert np.all(p_g[off[:-1][np.diff(off) > 0]] == 1.0)
    keep = np.abs(p_o - threshold) > 1e-5
    assert np.array_equal(b_g[keep], oracle.boundary_mask(p_o, threshold)[keep])
    assert float(to_np(tau)[0]) == np.float32(threshold)
    return p_g, b_g


def test_route_c0_fp32(ops):
    torch = _torch()
    c = gen_hnet_tiny()
    say("route tiny fp32", c["q"].shape)
    _check_route(ops, c["q"], c["k"], c["offsets"], torch.float32)


@pytest.mark.parametrize("d", [8, 64, 512, 768, 4096])
def test_route_ragged_bf16(ops, d):
    torch = _torch()
    rng = np.random.default_rng(100 + d)
    off, q, k, _ = _ragged(rng, [1, 0, 37, 300, 0, 1025, 2], d, torch.bfloat16)
    say("route ragged bf16 d", d, "N", off[-1])
    _check_route(ops, q, k, off, torch.bfloat16)


def test_route_zero_rows_and_nan(ops):
    torch = _torch()
    q = np.zeros((6, 8), np.float32); k = np.zeros((6, 8), np.float32)
    q[2] = 1.0; k[1] = 1.0                     # p_2: parallel -> 0
    q[3, 0] = np.nan                           # NaN -> b = 0
    off = np.array([0, 6], np.int64)
    p, b, _ = ops.route(to_dev(q), to_dev(k), to_dev(off), threshold=0.5)
    p, b = to_np(p), to_np(b)
    assert p[0] == 1.0 and p[1] == 0.5 and p[2] == 0.0 and np.isnan(p[3]) and b[3] == 0
    assert p[4] == 0.5 and b[4] == 1


def test_route_quantile_event_streams(ops):
    torch = _torch()
    c = gen_event_streams(nseq=6, d=512, min_events=3, max_events=40)
    say("route quantile event streams N", c["offsets"][-1])
    p, b, tau = ops.route(to_dev(c["q"], torch.bfloat16), to_dev(c["k"], torch.bfloat16),
                          to_dev(c["offsets"]), quantile=0.75)
    p_g, b_g, tau_g = to_np(p), to_np(b).astype(bool), float(to_np(tau)[0])
    n = len(p_g)
    assert tau_g == np.sort(p_g)[int(np.floor(0.75 * (n - 1)))]  # exact order statistic
    assert np.array_equal(b_g, p_g >= np.float32(tau_g))
    p_o = oracle.route(c["q"], c["k"], c["offsets"])
    assert abs(tau_g - oracle.stage_quantile(p_o, 0.75)) < 1e-5
    assert abs(b_g.mean() - 0.25) < 0.01


def test_route_quantile_extremes(ops):
    torch = _torch()
    rng = np.random.default_rng(7)
    off, q, k, _ = _ragged(rng, [50, 70], 16, torch.float32)
    for qt in (0.0, 1.0):
        p, b, tau = ops.route(to_dev(q), to_dev(k), to_dev(off), quantile=qt)
        p_g = to_np(p)
        want = p_g.min() if qt == 0.0 else p_g.max()
        assert float(to_np(tau)[0]) == want


def _check_quantile(p, b, tau, qt):
    """tau is the exact order statistic of the returned scores (NaN last) and b = [p >= tau]."""
    p_g, b_g, tau_g = to_np(p), to_np(b).astype(bool), float(to_np(tau)[0])
    n = len(p_g)
    want = np.sort(p_g)[int(np.floor(qt * (n - 1)))]
    assert tau_g == want or (np.isnan(tau_g) and np.isnan(want))
    assert np.array_equal(b_g, p_g >= np.float32(tau_g))
    return p_g, tau_g


def test_route_quantile_more_tiles_than_workgroups(ops):
    """Over 2^18 scores the select kernel re-reads its tiles on every digit;
    NaN scores sort last and are never kept."""
    torch = _torch()
    rng = np.random.default_rng(11)
    off, q, k, _ = _ragged(rng, [150_000, 1, 150_000, 37_123], 8, torch.float32)
    say("route quantile many tiles N", off[-1])
    p_o = oracle.route(q, k, off)
    for qt in (0.1, 0.75):
        p, b, tau = ops.route(to_dev(q), to_dev(k), to_dev(off), quantile=qt)
        _, tau_g = _check_quantile(p, b, tau, qt)
        assert abs(tau_g - oracle.stage_quantile(p_o, qt)) < 1e-5
    q[rng.integers(1, len(q), 100)] = np.nan
    p, b, tau = ops.route(to_dev(q), to_dev(k), to_dev(off), quantile=0.999)
    p_g, tau_g = _check_quantile(p, b, tau, 0.999)
    assert np.isnan(p_g).sum() > 50 and not np.isnan(tau_g)


def test_route_quantile_crowded_scores(ops):
    """Every non-start score is exactly 1/2 (q_t orthogonal to k_{t-1}), so
    all keys share one bin on every digit; a rank among the NaN scores gives
    tau = NaN and b = 0."""
    N, d = 70_000, 16
    q = np.zeros((N, d), np.float32); q[:, 0] = 1.0
    k = np.zeros((N, d), np.float32); k[:, 1] = 3.0
    off = np.array([0, 30_000, N], np.int64)
    for qt in (0.0, 0.5, 1.0):
        p, b, tau = ops.route(to_dev(q), to_dev(k), to_dev(off), quantile=qt)
        p_g, tau_g = _check_quantile(p, b, tau, qt)
        assert tau_g == (1.0 if qt == 1.0 else 0.5)
    q[5:] = np.nan
    p, b, tau = ops.route(to_dev(q), to_dev(k), to_dev(off), quantile=1.0)
    _, tau_g = _check_quantile(p, b, tau, 1.0)
    assert np.isnan(tau_g) and not to_np(b).any()


# ---------------------------------------------------------------- fused projection + route

def _fused_oracle(h, wq, wk, off):
    """The plain definition: q = h Wq, k = h Wk in fp64 from the bf16 inputs, then the route."""
    h64 = np.asarray(h, np.float64)
    return oracle.route(h64 @ np.asarray(wq, np.float64), h64 @ np.asarray(wk, np.float64), off)


@pytest.mark.parametrize("d", [128, 512, 768])
def test_route_fused_matches_oracle(ops, d):
    torch = _torch()
    bf = torch.bfloat16
    rng = np.random.default_rng(50 + d)
    off = np.concatenate([[0], np.cumsum([1, 0, 127, 128, 129, 900, 2])]).astype(np.int64)
    N = int(off[-1])
    h = bf16_round(rng.standard_normal((N, d)))
    wq = bf16_round(rng.standard_normal((d, d)) / np.sqrt(d))
    wk = bf16_round(rng.standard_normal((d, d)) / np.sqrt(d))
    p, b, tau = ops.route_fused(to_dev(h, bf), to_dev(wq, bf), to_dev(wk, bf), to_dev(off), threshold=0.5)
    p_g, b_g = to_np(p), to_np(b).astype(bool)
    p_o = _fused_oracle(h, wq, wk, off)
    say("route fused d", d, "N", N, "max |dp|", float(np.max(np.abs(p_g - p_o))))
    assert np.max(np.abs(p_g - p_o)) < 1e-5
    assert np.all(p_g[off[:-1][np.diff(off) > 0]] == 1.0)
    keep = np.abs(p_o - 0.5) > 1e-5
    assert np.array_equal(b_g[keep], (p_o >= 0.5)[keep])
    assert float(to_np(tau)[0]) == 0.5


def test_route_fused_largest_d(ops):
    """The largest supported width, d = 4096 (32 column blocks of q and k)."""
    torch = _torch()
    bf = torch.bfloat16
    d = 4096
    rng = np.random.default_rng(4096)
    off = np.array([0, 129, 130, 300], np.int64)
    N = int(off[-1])
    h = bf16_round(rng.standard_normal((N, d)))
    wq = bf16_round(rng.standard_normal((d, d)) / np.sqrt(d))
    wk = bf16_round(rng.standard_normal((d, d)) / np.sqrt(d))
    say("route fused d 4096")
    p, b, tau = ops.route_fused(to_dev(h, bf), to_dev(wq, bf), to_dev(wk, bf), to_dev(off), threshold=0.5)
    p_o = _fused_oracle(h, wq, wk, off)
    assert np.max(np.abs(to_np(p) - p_o)) < 1e-5
    keep = np.abs(p_o - 0.5) > 1e-5
    assert np.array_equal(to_np(b).astype(bool)[keep], (p_o >= 0.5)[keep])


def test_route_fused_quantile_event_streams(ops):
    """Stage-1 routing from h on ByteGen-style streams (projections formed in
    the kernel), with the stage's 0.75 score quantile."""
    torch = _torch()
    bf = torch.bfloat16
    c = gen_event_streams(nseq=6, d=512, min_events=3, max_events=40)
    off = c["offsets"]
    p, b, tau = ops.route_fused(to_dev(c["h"], bf), to_dev(c["wq"], bf), to_dev(c["wk"], bf), to_dev(off),
                                quantile=0.75)
    p_g, tau_g = _check_quantile(p, b, tau, 0.75)
    p_o = _fused_oracle(c["h"], c["wq"], c["wk"], off)
    assert np.max(np.abs(p_g - p_o)) < 1e-5
    assert abs(tau_g - oracle.stage_quantile(p_o, 0.75)) < 1e-5


def _compact_check(ops, b, p, rows, off, dtype, capacity=None):
    idx, coff, z, P, st = ops.compact(to_dev(b.astype(np.uint8)), to_dev(off), rows=to_dev(rows, dtype),
                                      p=to_dev(p.astype(np.float32)), capacity=capacity)
    i_o, c_o, z_o, P_o = oracle.compact(b, p.astype(np.float32), rows, off)
    M = len(i_o)
    cap = len(b) if capacity is None else capacity
    m = min(M, cap)
    assert np.array_equal(to_np(coff), c_o)
    assert np.array_equal(to_np(idx)[:m], i_o[:m])
    assert np.array_equal(to_np(z)[:m], z_o[:m])
    assert np.array_equal(to_np(P)[:m], P_o[:m])
    return idx, coff, z, P, st


def test_compact_matches_oracle_bitexact(ops):
    torch = _torch()
    rng = np.random.default_rng(11)
    off, q, k, h = _ragged(rng, [5000, 1, 0, 4096, 3, 8191, 17], 64, torch.bfloat16)
    p, b = _check_route(ops, q, k, off, torch.bfloat16)
    say("compact N", off[-1], "M", b.sum())
    _, _, _, _, st = _compact_check(ops, b, p, h, off, torch.bfloat16)
    assert int(to_np(st)[0]) == 0


def test_compact_capacity_overflow_sets_status(ops):
    torch = _torch()
    rng = np.random.default_rng(12)
    off = np.array([0, 300, 1000], np.int64)
    b = rng.random(1000) < 0.5
    p = rng.random(1000).astype(np.float32)
    h = rng.standard_normal((1000, 16)).astype(np.float32)
    cap = int(b.sum()) - 5
    _, _, _, _, st = _compact_check(ops, b, p, h, off, torch.float32, capacity=cap)
    assert int(to_np(st)[0]) & 1


def test_compact_edges_no_start_boundary_and_empty(ops):
    torch = _torch()
    off = np.array([0, 0, 10, 10, 25, 25], np.int64)
    b = np.zeros(25, bool); b[[3, 4, 12, 24]] = True  # sequence 1 has no boundary at its start
    p = np.linspace(0, 1, 25).astype(np.float32)
    h = np.arange(25 * 8, dtype=np.float32).reshape(25, 8)
    _compact_check(ops, b, p, h, off, torch.float32)
    # no boundary at all
    _compact_check(ops, np.zeros(25, bool), p, h, off, torch.float32)


def test_empty_batch_through_the_chain(ops):
    """A batch whose sequences are all empty: route (threshold and quantile),
    compact, dechunk and its backward accept empty tensors (NULL data
    pointers) and produce empty outputs, chunk offsets of zeros and tau as
    set (the threshold, or NaN for a quantile of no scores)."""
    torch = _torch()
    off = to_dev(np.array([0, 0, 0], np.int64))
    e = to_dev(np.zeros((0, 64), np.float32))
    p, b, tau = ops.route(e, e, off, threshold=0.5)
    assert p.numel() == 0 and b.numel() == 0 and float(to_np(tau)[0]) == 0.5
    p, b, tau = ops.route(e, e, off, quantile=0.75)
    assert np.isnan(float(to_np(tau)[0]))
    eb = to_dev(np.zeros((0, 128), np.float32), torch.bfloat16)
    w = to_dev(np.zeros((128, 128), np.float32), torch.bfloat16)
    p, b, tau = ops.route_fused(eb, w, w, off, threshold=0.25)
    assert p.numel() == 0 and float(to_np(tau)[0]) == 0.25
    idx, coff, z, P, st = ops.compact(b, off, rows=e, p=p)
    assert np.array_equal(to_np(coff), [0, 0, 0]) and int(to_np(st)[0]) == 0
    out = ops.dechunk_ema(z, P, idx, coff, off, 0)
    assert out.shape == (0, 64)
    dz, dP = ops.dechunk_ema_backward(z[:0], P[:0], e, idx[:0], coff, off)
    assert dz.numel() == 0 and dP.numel() == 0


def _dechunk_check(ops, z, P, idx, coff, off, dtype, tol):
    N = int(off[-1])
    out = ops.dechunk_ema(to_dev(z, dtype), to_dev(P.astype(np.float32)), to_dev(idx.astype(np.int32)),
                          to_dev(coff), to_dev(off), N)
    ref = oracle.dechunk_ema(z, P.astype(np.float32), idx, coff, off)
    err = row_rel_err(to_np(out), ref)
    assert err < tol, err
    return out


@pytest.mark.parametrize("dtname,d", [("f32", 64), ("bf16", 512), ("bf16", 768), ("f32", 8), ("bf16", 4096)])
def test_dechunk_matches_oracle(ops, dtname, d):
    torch = _torch()
    dtype = torch.float32 if dtname == "f32" else torch.bfloat16
    rng = np.random.default_rng(20 + d)
    off, q, k, h = _ragged(rng, [3000, 1, 0, 5000, 64], d, dtype)
    p, b = _check_route(ops, q, k, off, dtype)
    idx, coff, z, P, _ = ops.compact(to_dev(b.astype(np.uint8)), to_dev(off), rows=to_dev(h, dtype),
                                     p=to_dev(p))
    M = int(to_np(coff)[-1])
    say("dechunk", dtname, d, "N", off[-1], "M", M)
    _dechunk_check(ops, to_np(z)[:M], to_np(P)[:M], to_np(idx)[:M].astype(np.int64), to_np(coff), off,
                   dtype, 1e-4 if dtname == "f32" else 2e-2)


def test_dechunk_identity_when_P_is_one(ops):
    torch = _torch()
    rng = np.random.default_rng(31)
    for dtype in (torch.float32, torch.bfloat16):
        off = np.array([0, 17, 17, 4000, 9001], np.int64)
        N = 9001
        rows = rng.standard_normal((N, 32)).astype(np.float32)
        rows_t = to_dev(rows, dtype)
        idx = np.arange(N, dtype=np.int32)
        out = ops.dechunk_ema(rows_t, to_dev(np.ones(N, np.float32)), to_dev(idx), to_dev(off), to_dev(off), N)
        assert torch.equal(out, rows_t)


def test_dechunk_many_chunks_and_zero_prefix(ops):
    torch = _torch()
    rng = np.random.default_rng(32)
    # > 4096 chunks so tiles hold several chunks; sequences that start without a boundary
    off = np.array([0, 9000, 9000, 20000], np.int64)
    b = rng.random(20000) < 0.6
    b[0] = False; b[:5] = False; b[9000] = False; b[9000:9010] = False
    P = rng.uniform(0.05, 1.0, 20000).astype(np.float32)
    rows = rng.standard_normal((20000, 16)).astype(np.float32)
    idx, coff, z, PP = oracle.compact(b, P, rows, off)
    out = _dechunk_check(ops, z, PP, idx, coff, off, torch.float32, 1e-4)
    assert np.all(to_np(out)[:5] == 0) and np.all(to_np(out)[9000:9010] == 0)
    # no chunks at all: everything zero
    e = np.zeros(0, np.int64)
    o2 = ops.dechunk_ema(to_dev(np.zeros((1, 16), np.float32)), to_dev(np.zeros(1, np.float32)),
                         to_dev(np.zeros(1, np.int32)), to_dev(np.zeros(4, np.int64)), to_dev(off), 20000)
    assert float(o2.abs().max()) == 0.0


def test_dechunk_many_short_sequences(ops):
    """700 ragged sequences (some empty, some without a boundary at their
    start): resets inside most scan units, many sequences per zeroing block."""
    torch = _torch()
    rng = np.random.default_rng(33)
    lengths = rng.integers(0, 41, 700)
    lengths[::7] = 0
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = int(off[-1])
    b = rng.random(N) < 0.3
    starts = off[:-1][lengths > 0]
    b[starts[::2]] = True
    P = rng.uniform(0.0, 1.0, N).astype(np.float32)
    rows = rng.standard_normal((N, 24)).astype(np.float32)
    idx, coff, z, PP = oracle.compact(b, P, rows, off)
    say("dechunk many short sequences N", N, "M", len(idx))
    for dtype in (torch.float32, torch.bfloat16):
        _dechunk_check(ops, z, PP, idx, coff, off, dtype, 1e-4 if dtype == torch.float32 else 2e-2)


# ---------------------------------------------------------------- EMA backward

def _dechunk_bwd_check(ops, z, P, idx, coff, off, dout, dtype, tol):
    dz, dP = ops.dechunk_ema_backward(to_dev(z, dtype), to_dev(P.astype(np.float32)), to_dev(dout, dtype),
                                      to_dev(idx.astype(np.int32)), to_dev(coff), to_dev(off))
    if dtype != _torch().float32:
        from synthdata import bf16_round
        z, dout = bf16_round(z), bf16_round(dout)
    dz_o, dP_o = oracle.dechunk_ema_backward(z, P.astype(np.float32), idx, coff, off, dout)
    M = len(idx)
    dz_g, dP_g = to_np(dz)[:M], to_np(dP)[:M]
    scale = max(np.max(np.abs(dP_o)), 1e-30)
    say("dechunk backward", z.shape[1], "dz max row rel err", row_rel_err(dz_g, dz_o), "dP max err / max |dP|",
        np.max(np.abs(dP_g - dP_o)) / scale)
    assert row_rel_err(dz_g, dz_o) < tol
    assert np.max(np.abs(dP_g - dP_o)) / scale < tol, np.max(np.abs(dP_g - dP_o)) / scale
    return dz_g, dP_g


@pytest.mark.parametrize("dtname,d", [("f32", 64), ("bf16", 512), ("bf16", 768), ("f32", 8), ("bf16", 2048)])
def test_dechunk_backward_matches_oracle(ops, dtname, d):
    torch = _torch()
    dtype = torch.float32 if dtname == "f32" else torch.bfloat16
    rng = np.random.default_rng(40 + d)
    off = np.array([0, 3000, 3001, 3001, 8000, 8064], np.int64)
    N = int(off[-1])
    b = rng.random(N) < 0.3
    b[[0, 3000, 3001, 8000]] = True
    b[8000:8010] = False   # a sequence without a boundary at its start
    P = rng.uniform(0.02, 1.0, N).astype(np.float32)
    rows = rng.standard_normal((N, d)).astype(np.float32)
    idx, coff, z, PP = oracle.compact(b, P, rows, off)
    dout = rng.standard_normal((N, d)).astype(np.float32)
    say("dechunk backward", dtname, d, "N", N, "M", len(idx))
    _dechunk_bwd_check(ops, z.astype(np.float32), PP, idx, coff, off, dout, dtype,
                       1e-4 if dtname == "f32" else 2e-2)


def test_dechunk_backward_P_one_is_dout(ops):
    """P = 1 at every position and every position a boundary: dz = dout bit for bit."""
    torch = _torch()
    rng = np.random.default_rng(41)
    for dtype in (torch.float32, torch.bfloat16):
        off = np.array([0, 17, 17, 4000, 9001], np.int64)
        N = 9001
        z = to_dev(rng.standard_normal((N, 32)).astype(np.float32), dtype)
        g = to_dev(rng.standard_normal((N, 32)).astype(np.float32), dtype)
        idx = to_dev(np.arange(N, dtype=np.int32))
        dz, dP = ops.dechunk_ema_backward(z, to_dev(np.ones(N, np.float32)), g, idx, to_dev(off), to_dev(off))
        assert torch.equal(dz, g)


def test_dechunk_backward_many_short_sequences(ops):
    """700 ragged sequences (some empty, some without a start boundary)."""
    torch = _torch()
    rng = np.random.default_rng(42)
    lengths = rng.integers(0, 41, 700)
    lengths[::7] = 0
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = int(off[-1])
    b = rng.random(N) < 0.3
    starts = off[:-1][lengths > 0]
    b[starts[::2]] = True
    P = rng.uniform(0.0, 1.0, N).astype(np.float32)
    rows = rng.standard_normal((N, 24)).astype(np.float32)
    idx, coff, z, PP = oracle.compact(b, P, rows, off)
    dout = rng.standard_normal((N, 24)).astype(np.float32)
    _dechunk_bwd_check(ops, z.astype(np.float32), PP, idx, coff, off, dout, torch.float32, 1e-4)


def test_dechunk_backward_full_size_stage1_sampled(ops):
    """Stage-1 backward at the bench.py size (32 x 8192 rows, 65.7k chunks x 512,
    bf16): two sequences checked against the oracle."""
    torch = _torch()
    bf = torch.bfloat16
    c = gen_hnet_two_stage(fixed_T=8192)
    off = c["offsets"]
    p = oracle.route(c["q"], c["k"], off)
    tau = oracle.stage_quantile(p, 0.75)
    b = oracle.boundary_mask(p, tau)
    idx, coff, z, P = oracle.compact(b, p.astype(np.float32), c["h"], off)
    rng = np.random.default_rng(43)
    N = int(off[-1])
    dout = bf16_round(rng.standard_normal((N, 512)).astype(np.float32))
    dz, dP = ops.dechunk_ema_backward(to_dev(z, bf), to_dev(P.astype(np.float32)), to_dev(dout, bf),
                                      to_dev(idx.astype(np.int32)), to_dev(coff), to_dev(off))
    dz, dP = to_np(dz), to_np(dP)
    for s in (0, 31):
        c0, c1 = int(coff[s]), int(coff[s + 1])
        t0, t1 = int(off[s]), int(off[s + 1])
        o_s = np.array([0, t1 - t0], np.int64)
        dz_o, dP_o = oracle.dechunk_ema_backward(z[c0:c1], P[c0:c1].astype(np.float32), idx[c0:c1] - t0,
                                                 np.array([0, c1 - c0], np.int64), o_s, dout[t0:t1])
        assert row_rel_err(dz[c0:c1], dz_o) < 2e-2
        assert np.max(np.abs(dP[c0:c1] - dP_o)) / np.max(np.abs(dP_o)) < 2e-2
    say("dechunk backward full size ok, M", len(idx))


@pytest.mark.parametrize("fixed_T", [8192, None], ids=["T8192", "ragged"])
def test_c2_two_stage_full_size(ops, fixed_T):
    """The two-stage H-Net workload at full size: 32 streams (every one 8192
    bytes, the launch configuration of bench.py, or ragged lengths of 32 x
    U{32..256} events up to 8192 bytes), two stages at the 0.75 score quantile
    each, both EMA scans back to full length."""
    torch = _torch()
    bf = torch.bfloat16
    c = gen_hnet_two_stage(fixed_T=fixed_T)
    off = c["offsets"]; N = int(off[-1])
    say("two-stage 32 streams generated, fixed_T", fixed_T, "N", N)
    p1, b1, tau1 = ops.route(to_dev(c["q"], bf), to_dev(c["k"], bf), to_dev(off), quantile=0.75)
    p1g, b1g = to_np(p1), to_np(b1).astype(bool)
    p1o = oracle.route(c["q"], c["k"], off)
    assert np.max(np.abs(p1g - p1o)) < 5e-6
    tau1g = float(to_np(tau1)[0])
    assert tau1g == np.sort(p1g)[int(np.floor(0.75 * (N - 1)))]
    assert abs(tau1g - oracle.stage_quantile(p1o, 0.75)) < 1e-5
    idx1, coff1, z1, P1, st = ops.compact(b1, to_dev(off), rows=to_dev(c["h"], bf), p=p1)
    i1o, c1o, z1o, P1o = oracle.compact(b1g, p1g, c["h"], off)
    M1 = len(i1o)
    assert np.array_equal(to_np(coff1), c1o) and np.array_equal(to_np(idx1)[:M1], i1o)
    assert np.array_equal(to_np(z1)[:M1], z1o) and np.array_equal(to_np(P1)[:M1], P1o)
    say("stage 1 M1", M1, "ratio", M1 / N)
    s2 = gen_stage2_inputs(z1o, c)
    p2, b2, tau2 = ops.route(to_dev(s2["q2"], bf), to_dev(s2["k2"], bf), coff1, quantile=0.75)
    p2g, b2g = to_np(p2), to_np(b2).astype(bool)
    p2o = oracle.route(s2["q2"], s2["k2"], c1o)
    assert np.max(np.abs(p2g - p2o)) < 5e-6
    idx2, coff2, z2, P2, _ = ops.compact(b2, coff1, rows=to_dev(s2["x2"], bf), p=p2)
    i2o, c2o, z2o, P2o = oracle.compact(b2g, p2g, s2["x2"], c1o)
    M2 = len(i2o)
    assert np.array_equal(to_np(idx2)[:M2], i2o) and np.array_equal(to_np(z2)[:M2], z2o)
    say("stage 2 M2", M2, "ratio", M2 / N)
    assert 0.2 < M1 / N < 0.3 and 0.04 < M2 / N < 0.09
    y2 = ops.dechunk_ema(z2, P2, idx2, coff2, coff1, M1)
    y2o = oracle.dechunk_ema(z2o, P2o, i2o, c2o, c1o)
    assert row_rel_err(to_np(y2), y2o) < 2e-2
    y1 = gen_stage2_backproj(to_np(y2), c)
    out = ops.dechunk_ema(to_dev(y1, bf), P1, idx1, coff1, to_dev(off), N)
    outo = oracle.dechunk_ema(y1, P1o, i1o, c1o, off)
    assert row_rel_err(to_np(out), outo) < 2e-2
    say("two-stage chain ok")


def test_c1_event_streams_chain_full_size(ops):
    """The ByteGen-style workload at full size: 16 ragged streams of 32 x
    U{32..256} events, d 512 bf16, threshold 0.5: route, compact and EMA
    dechunk of the compacted rows back to byte length, every position and row
    against the oracle."""
    torch = _torch()
    bf = torch.bfloat16
    c = gen_event_streams()
    off = c["offsets"]; N = int(off[-1])
    say("event streams generated N", N, "lengths", np.diff(off).min(), np.diff(off).max())
    p, b, tau = ops.route(to_dev(c["q"], bf), to_dev(c["k"], bf), to_dev(off), threshold=0.5)
    p_g, b_g = to_np(p), to_np(b).astype(bool)
    p_o = oracle.route(c["q"], c["k"], off)
    assert np.max(np.abs(p_g - p_o)) < 5e-6
    keep = np.abs(p_o - 0.5) > 1e-5
    assert np.array_equal(b_g[keep], oracle.boundary_mask(p_o, 0.5)[keep])
    idx, coff, z, P, st = ops.compact(b, to_dev(off), rows=to_dev(c["h"], bf), p=p)
    i_o, c_o, z_o, P_o = oracle.compact(b_g, p_g, c["h"], off)
    M = len(i_o)
    say("M", M, "ratio", M / N)
    assert int(to_np(st)[0]) == 0
    assert np.array_equal(to_np(coff), c_o) and np.array_equal(to_np(idx)[:M], i_o)
    assert np.array_equal(to_np(z)[:M], z_o) and np.array_equal(to_np(P)[:M], P_o)
    out = ops.dechunk_ema(z, P, idx, coff, to_dev(off), N)
    ref = oracle.dechunk_ema(z_o, P_o, i_o, c_o, off)
    assert row_rel_err(to_np(out), ref) < 2e-2
    say("event-stream chain ok")


def test_dechunk_after_capacity_overflow_stays_in_bounds(ops):
    """A compaction whose capacity is below the boundary count flags
    BLLM_S_CAPACITY and keeps the true counts in its chunk offsets; the EMA
    dechunk and its backward given max_chunks = capacity use only the stored
    chunks (offsets clamped to the capacity: the sequence cut short keeps its
    last stored chunk to its end, later sequences get zero rows) and never
    touch rows past the capacity, which hold sentinel values here."""
    torch = _torch()
    rng = np.random.default_rng(77)
    lengths = np.array([40, 0, 55, 33, 61], np.int64)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N, d = int(off[-1]), 16
    b = rng.random(N) < 0.5
    b[off[:-1][lengths > 0]] = True
    p = rng.uniform(0.05, 1.0, N).astype(np.float32)
    h = rng.standard_normal((N, d)).astype(np.float32)
    M = int(b.sum())
    i_o, c_o, z_o, P_o = oracle.compact(b, p, h, off)
    cap = int(c_o[3]) - 2  # drops the last two chunks of sequence 2 and all chunks after it
    assert c_o[2] < cap
    # outputs larger than the capacity, the rows past it filled with sentinels
    # (idx 0 is a valid position: a read past the capacity shows as a wrong result)
    idx_buf = torch.zeros((M,), dtype=torch.int32, device="cuda")
    rows_buf = torch.full((M, d), float("nan"), dtype=torch.float32, device="cuda")
    P_buf = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    idx, coff, z, P, st = ops.compact(to_dev(b.astype(np.uint8)), to_dev(off), rows=to_dev(h), p=to_dev(p),
                                      capacity=cap, idx_out=idx_buf, rows_out=rows_buf, P_out=P_buf)
    assert int(to_np(st)[0]) & 1
    assert np.array_equal(to_np(coff), c_o)  # true counts
    assert np.array_equal(to_np(idx)[:cap], i_o[:cap]) and np.all(to_np(idx)[cap:] == 0)
    cc = np.minimum(c_o, cap)
    out = ops.dechunk_ema(z, P, idx, coff, to_dev(off), N, max_chunks=cap)
    ref = oracle.dechunk_ema(z_o[:cap], P_o[:cap], i_o[:cap], cc, off)
    o = to_np(out)
    assert np.all(np.isfinite(o))
    assert row_rel_err(o, ref) < 1e-4
    dout = rng.standard_normal((N, d)).astype(np.float32)
    dz, dP = ops.dechunk_ema_backward(z, P, to_dev(dout), idx, coff, to_dev(off), max_chunks=cap)
    dz_o, dP_o = oracle.dechunk_ema_backward(z_o[:cap], P_o[:cap], i_o[:cap], cc, off, dout)
    dz, dP = to_np(dz), to_np(dP)
    assert dz.shape[0] == cap and np.all(np.isfinite(dz)) and np.all(np.isfinite(dP))
    assert row_rel_err(dz, dz_o) < 1e-4
    assert np.max(np.abs(dP - dP_o)) <= 1e-4 * max(1.0, np.max(np.abs(dP_o)))
    # no stored chunk at all: every output row is zero
    out0 = ops.dechunk_ema(z, P, idx, coff, to_dev(off), N, max_chunks=0)
    assert np.all(to_np(out0) == 0)


def test_route_quantile_reports_a_wait_that_gave_up(ops):
    """The stage quantile's bounded grid-wide waits: the library built with a
    spin limit of 0 (every wait gives up at once; every kernel still exits
    normally) ORs BLLM_S_INCOMPLETE into the status word and returns tau = NaN;
    the real library leaves the word clear on the same input."""
    import ctypes as C
    import os
    torch = _torch()
    from byte_level_lm_amd import _lib as L
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "libbllm_spin0.so")
    assert os.path.exists(path), f"{path} not built: run __graft_entry__.build()"
    spin0 = C.CDLL(path)
    spin0.bllm_route.restype = C.c_int
    spin0.bllm_route.argtypes = L._SIGS["bllm_route"][1]
    rng = np.random.default_rng(78)
    off, q, k, _ = _ragged(rng, [5000, 7000, 9000], 64, torch.float32)
    N = int(off[-1])
    qd, kd, od = to_dev(q), to_dev(k), to_dev(off)
    for lib, want in ((spin0, L.S_INCOMPLETE), (L.lib(), 0)):
        p = torch.empty(N, device="cuda"); b = torch.empty(N, dtype=torch.uint8, device="cuda")
        tau = torch.empty(1, device="cuda"); st = torch.zeros(1, dtype=torch.int32, device="cuda")
        ws = torch.empty(ops.route_workspace(N), dtype=torch.uint8, device="cuda")
        rc = lib.bllm_route(qd.data_ptr(), kd.data_ptr(), L.F32, 64, od.data_ptr(), 3, N, 0.5, 0.75,
                            p.data_ptr(), b.data_ptr(), tau.data_ptr(), st.data_ptr(), ws.data_ptr(),
                            ws.numel(), torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        assert int(to_np(st)[0]) == want
        t = float(to_np(tau)[0])
        assert np.isnan(t) if want else t == np.sort(to_np(p))[int(np.floor(0.75 * (N - 1)))]
