"""GPU parity: ByteFlow coding rate, Top-K, gather and binned upsample against the oracle."""
import numpy as np
import pytest

import oracle
from synthdata import (bf16_round, cluster_rows, gen_coding_rate_tiny, gen_coding_rate_fp32, gen_byteflow_layer,
                       gen_global_standin, gen_cosine_qk)
from tests.helpers import oracle_dr_parallel, row_rel_err, say, to_dev, to_np, topk_band_compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import byte_level_lm_amd as B
    B.lib()
    return B


def _torch():
    import torch
    return torch


# ------------------------------------------------------------------ Top-K

def _topk_check(ops, sc, K):
    idx, mask, st = ops.topk_select(to_dev(sc.astype(np.float32)), K)
    want = oracle.topk_select(sc.astype(np.float32), K)
    assert np.array_equal(to_np(idx), want)
    assert np.array_equal(to_np(mask), oracle.topk_mask(want, sc.shape[1]))
    return st


def test_topk_bitexact_on_oracle_delta_r(ops):
    rng = np.random.default_rng(1)
    h = cluster_rows(rng, 2, 600, 16)
    dr = oracle.coding_rate(h, 0.5).astype(np.float32)
    for K in (1, 2, 3, 150, 599, 600):
        _topk_check(ops, dr, K)


def test_topk_ties_specials_and_ragged_sizes(ops):
    rng = np.random.default_rng(2)
    for T in (1, 2, 5, 1023, 1025, 3000, 16384):
        sc = rng.integers(0, 5, size=(3, T)).astype(np.float32)
        sc[0, ::7] = -0.0
        sc[1, ::11] = np.inf
        sc[2, ::13] = -np.inf
        for K in sorted({1, min(T, 2), max(1, T // 3), T}):
            _topk_check(ops, sc, K)
    sc = rng.standard_normal((2, 100)).astype(np.float32)
    sc[0, 5] = np.nan
    st = _topk_check(ops, sc, 30)
    assert int(to_np(st)[0]) & 2


def test_topk_long_sequences_from_memory(ops):
    """Past 16384 positions the keys are recomputed from the scores in every
    radix pass (up to 64 positions per thread): ties, signed zeros, +-inf and
    a NaN, then real-valued scores, at lengths across that switch."""
    rng = np.random.default_rng(4)
    for T in (16385, 32768, 40000, 65536):
        sc = rng.integers(0, 7, size=(2, T)).astype(np.float32)
        sc[0, ::7] = -0.0
        sc[1, ::11] = np.inf
        sc[1, 3::13] = -np.inf
        for K in (1, 2, T // 4, T - 1, T):
            _topk_check(ops, sc, K)
    sc = rng.standard_normal((3, 65536)).astype(np.float32)
    sc[2, 1000] = np.nan
    st = _topk_check(ops, sc, 8192)
    assert int(to_np(st)[0]) & 2


def test_topk_full_size_c3_shape(ops):
    rng = np.random.default_rng(3)
    sc = rng.standard_normal((8, 8192)).astype(np.float32)
    _topk_check(ops, sc, 2048)


# ------------------------------------------------------------------ coding rate

def _dr(ops, h, eps2, dtype):
    dR, st = ops.coding_rate(to_dev(h, dtype), eps2)
    return to_np(dR), int(to_np(st)[0])


def test_coding_rate_tiny_brute_force_case(ops):
    torch = _torch()
    c = gen_coding_rate_tiny()
    g, st = _dr(ops, c["h"][None], c["eps2"], torch.float32)
    o = oracle.coding_rate(c["h"], c["eps2"])
    assert st == 0
    assert np.max(np.abs(g[0] - o) / np.abs(o)) < 1e-4


@pytest.mark.parametrize("T,d", [(700, 64), (1000, 256), (33, 8), (129, 40)])
def test_coding_rate_fp32_vs_oracle(ops, T, d):
    torch = _torch()
    rng = np.random.default_rng(T + d)
    h = cluster_rows(rng, 2, T, d).astype(np.float32)
    say("coding_rate fp32 T", T, "d", d)
    g, st = _dr(ops, h, 0.5, torch.float32)
    assert st == 0
    for s in range(2):
        o = oracle.coding_rate(h[s], 0.5)
        assert np.max(np.abs(g[s] - o) / np.abs(o)) < 1e-3


def test_coding_rate_bf16_d512_vs_oracle(ops):
    torch = _torch()
    rng = np.random.default_rng(5)
    h = bf16_round(cluster_rows(rng, 1, 600, 512))
    say("coding_rate bf16 d=512 T=600")
    g, st = _dr(ops, h, 0.5, torch.bfloat16)
    o = oracle_dr_parallel(h[0].astype(np.float64), 0.5)
    assert st == 0
    assert np.max(np.abs(g[0] - o) / np.abs(o)) < 1e-3


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_coding_rate_largest_d(ops, dt):
    """The largest supported width, d = 640 (ten 64-wide tiles, block
    matrices of 640 + 256), whole sequence and two streamed windows."""
    torch = _torch()
    rng = np.random.default_rng(640)
    h = cluster_rows(rng, 1, 400, 640)
    h = bf16_round(h) if dt == "bf16" else h.astype(np.float32)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    say("coding_rate d 640", dt)
    g, st = _dr(ops, h, 0.5, tdt)
    assert st == 0
    o = oracle.coding_rate(h[0].astype(np.float64), 0.5)
    assert np.max(np.abs(g[0] - o) / np.abs(o)) < 1e-3
    gs, A = _stream(ops, h, 0.5, tdt, (150, 250), inplace=True)
    assert np.max(np.abs(gs[0] - o) / np.abs(o)) < 1e-3
    want = np.eye(640) + oracle.alpha_of(640, 0.5) * h[0].astype(np.float64).T @ h[0].astype(np.float64)
    assert np.max(np.abs(A[0] - want)) <= 1e-5 * np.max(np.abs(want))


@pytest.mark.parametrize("T", [1, 2, 65])
def test_coding_rate_shortest_sequences(ops, T):
    """One- and two-row sequences (a single partial block), and one row past a
    64-row tile; the first value is R(h_1) = 1/2 log(1 + alpha |h_1|^2)."""
    torch = _torch()
    rng = np.random.default_rng(60 + T)
    h = cluster_rows(rng, 3, T, 64).astype(np.float32)
    g, st = _dr(ops, h, 0.5, torch.float32)
    assert st == 0
    a = oracle.alpha_of(64, 0.5)
    first = 0.5 * np.log1p(a * (h[:, 0].astype(np.float64) ** 2).sum(1))
    assert np.max(np.abs(g[:, 0] - first) / first) < 1e-5
    for s in range(3):
        o = oracle.coding_rate(h[s], 0.5)
        assert np.max(np.abs(g[s] - o) / np.abs(o)) < 1e-3


def test_coding_rate_nonfinite_sets_status(ops):
    torch = _torch()
    h = cluster_rows(np.random.default_rng(6), 1, 100, 16).astype(np.float32)
    h[0, 50, 3] = np.nan
    _, st = _dr(ops, h, 0.5, torch.float32)
    assert st & 2


def _near_cut_error(g, o, K, width=1e-4):
    """max |Delta R_gpu - Delta R_oracle| over positions within `width` of the
    oracle's K-th value (the values that decide the Top-K set)."""
    vK = np.sort(o[1:])[::-1][K - 2]
    near = np.abs(o - vK) <= width
    return float(np.max(np.abs(g[near] - o[near]))) if near.any() else 0.0, int(near.sum())


def _topk_sets_vs_oracle(ops, g, H, eps2, K, seqs, tag):
    """Every listed sequence: all Delta R within 1e-3 relative of the oracle,
    the Top-K set equal to the oracle's outside the 1e-5 band around the K-th
    value, and the error near the cut small enough (< 5e-6, half the band)
    that no position outside the band can change sides."""
    import torch
    idx, _, _ = ops.topk_select(to_dev(g), K)
    idx = to_np(idx)
    worst = 0.0
    for s_ in seqs:
        o = oracle_dr_parallel(H[s_].astype(np.float64), eps2)
        assert np.max(np.abs(g[s_] - o) / o) < 1e-3, s_
        bad, nband = topk_band_compare(idx[s_], oracle.topk_select(o, K), o, K)
        near, nnear = _near_cut_error(g[s_], o, K)
        worst = max(worst, near)
        say(tag, "seq", s_, "max abs err", float(np.max(np.abs(g[s_] - o))), "near-cut err", near,
            "positions within 1e-4", nnear, "band", nband, "flips", len(bad))
        assert len(bad) == 0, (s_, bad)
        assert near < 5e-6, (s_, near)
    say(tag, "worst near-cut error", worst, "over", len(seqs), "sequences")


def test_coding_rate_topk_full_size_fp32_8x8192x256(ops):
    """Full size: 8 x 8192 x 256 fp32.  Every sequence's Delta R against the
    oracle and its Top-K set (K = 2048) outside the 1e-5 band."""
    torch = _torch()
    c = gen_coding_rate_fp32()
    say("fp32 8 x 8192 x 256 generated")
    g, st = _dr(ops, c["h"], c["eps2"], torch.float32)
    assert st == 0
    _topk_sets_vs_oracle(ops, g, c["h"], c["eps2"], c["K"], range(c["nseq"]), "fp32")


def test_coding_rate_full_size_bf16_32x8192x512(ops):
    """Full size: 32 x 8192 x 512 bf16 (the launch configuration of bench.py).
    Eight of the 32 sequences (every fourth) against the oracle in full:
    Delta R within 1e-3 relative and the Top-K set outside the 1e-5 band."""
    torch = _torch()
    c = gen_byteflow_layer()
    say("bf16 32 x 8192 x 512 generated")
    g, st = _dr(ops, c["h"], c["eps2"], torch.bfloat16)
    assert st == 0
    _topk_sets_vs_oracle(ops, g, c["h"], c["eps2"], c["K"], range(0, 32, 4), "bf16")


@pytest.mark.parametrize("dt,nseq,T,d", [("f32", 3, 11000, 64), ("bf16", 2, 65536, 512)])
def test_coding_rate_batch_matches_single_sequences(ops, dt, nseq, T, d):
    """Batches of 512 or more row blocks (3 sequences with a ragged last
    block; 2 sequences of 256 blocks): each sequence's Delta R equals, bit for
    bit, a call on that sequence alone, and sampled positions of the last
    sequence match the oracle."""
    torch = _torch()
    rng = np.random.default_rng(50 + d)
    h = cluster_rows(rng, nseq, T, d)
    h = bf16_round(h) if dt == "bf16" else h.astype(np.float32)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    say("batch", nseq, "x", T, "x", d, dt)
    g, st = _dr(ops, h, 0.5, tdt)
    assert st == 0
    for s in range(nseq):
        one, st1 = _dr(ops, h[s:s + 1], 0.5, tdt)
        assert st1 == 0
        assert np.array_equal(g[s], one[0]), s
    if d <= 64:
        pos = np.sort(np.concatenate([[0, T - 1], rng.choice(T, 6, replace=False)]))
        o = oracle.coding_rate_at(h[-1], 0.5, pos)
        assert np.max(np.abs(g[-1, pos] - o) / np.abs(o)) < 1e-3



@pytest.mark.parametrize("dt,nseq,T,d", [("f32", 3, 11000, 64), ("bf16", 32, 8192, 512)])
def test_coding_rate_split_equals_one_stream(ops, dt, nseq, T, d):
    """The batch split over the caller's two streams (3 sequences: 2 + 1 with a
    ragged last block; the full 32 x 8192 x 512 bf16 workload, 16 + 16):
    bit-identical to the one-stream call, read after synchronising only the
    caller's stream."""
    torch = _torch()
    rng = np.random.default_rng(63 + d)
    h = cluster_rows(rng, nseq, T, d)
    h = bf16_round(h) if dt == "bf16" else h.astype(np.float32)
    hd = to_dev(h, torch.bfloat16 if dt == "bf16" else torch.float32)
    say("split vs one stream", nseq, "x", T, "x", d, dt)
    one, st1 = ops.coding_rate(hd, 0.5)
    torch.cuda.synchronize()
    s2, fe, je = torch.cuda.Stream(), torch.cuda.Event(), torch.cuda.Event()
    for rep in range(2):
        two, st2 = ops.coding_rate_split(hd, 0.5, s2, fe, je)
        torch.cuda.current_stream().synchronize()
        assert np.array_equal(to_np(two), to_np(one)), rep
        assert int(to_np(st2)[0]) == 0 and int(to_np(st1)[0]) == 0


def test_coding_rate_split_in_a_captured_graph(ops):
    """The two-stream form captured in a HIP graph (the fork and join events
    recorded inside the capture): replays with new inputs equal the eager
    one-stream result bit for bit."""
    torch = _torch()
    rng = np.random.default_rng(64)
    hs = [cluster_rows(rng, 2, 16384, 64).astype(np.float32) for _ in range(2)]
    want = [_dr(ops, h, 0.5, torch.float32)[0] for h in hs]
    hd = to_dev(hs[0], torch.float32)
    s2, fe, je = torch.cuda.Stream(), torch.cuda.Event(), torch.cuda.Event()
    ops.coding_rate_split(hd, 0.5, s2, fe, je)  # creates the events before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out, st = ops.coding_rate_split(hd, 0.5, s2, fe, je)
    for r in range(4):
        i = r % 2
        hd.copy_(torch.from_numpy(hs[i]).to(hd.device))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say("split graph replay", r)
        assert np.array_equal(to_np(out), want[i]), r
        assert int(to_np(st)[0]) == 0
        _dr(ops, hs[1 - i][:1, :4096], 0.5, torch.float32)  # eager work between replays


def test_coding_rate_in_a_captured_graph(ops):
    """A coding-rate call captured in a HIP graph (no warm-up call needed: the
    library keeps no state); replays with new inputs copied in, eager work and
    synchronisations between them, each equal the eager result bit for bit."""
    torch = _torch()
    rng = np.random.default_rng(60)
    hs = [cluster_rows(rng, 2, 16384, 64).astype(np.float32) for _ in range(2)]  # 2 x 256 blocks
    want = [_dr(ops, h, 0.5, torch.float32)[0] for h in hs]
    hd = to_dev(hs[0], torch.float32)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out, st = ops.coding_rate(hd, 0.5)
    for r in range(4):
        i = r % 2
        hd.copy_(torch.from_numpy(hs[i]).to(hd.device))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say("graph replay", r)
        assert np.array_equal(to_np(out), want[i]), r
        assert int(to_np(st)[0]) == 0
        _dr(ops, hs[1 - i][:1, :4096], 0.5, torch.float32)  # eager work between replays



def test_coding_rate_from_two_host_threads(ops):
    """Two host threads, each on a stream of its own, queue large batches at
    the same time: every result equals the same call made alone."""
    import threading
    torch = _torch()
    rng = np.random.default_rng(61)
    hs = [cluster_rows(rng, 2, 16384, 64).astype(np.float32) for _ in range(2)]  # 2 x 256 blocks each
    want = [_dr(ops, h, 0.5, torch.float32)[0] for h in hs]
    hd = [to_dev(h, torch.float32) for h in hs]
    torch.cuda.synchronize()
    got = [[None] * 3 for _ in range(2)]
    errs = []

    def run(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for r in range(3):
                    dR, status = ops.coding_rate(hd[i], 0.5)
                    got[i][r] = (dR, status)
            st.synchronize()
        except Exception as e:  # reported below, in the main thread
            errs.append(e)

    th = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errs, errs
    torch.cuda.synchronize()
    for i in range(2):
        for r in range(3):
            dR, status = got[i][r]
            assert np.array_equal(to_np(dR), want[i]), (i, r)
            assert int(to_np(status)[0]) == 0



def test_coding_rate_stream_batch_carries_state_per_sequence(ops):
    """Streaming windows of a batch (4 sequences x 16384-row windows, d 64:
    4 x 256 row blocks): the Delta R of both windows and the carried matrices
    equal, bit for bit, the same windows run for each sequence alone."""
    torch = _torch()
    rng = np.random.default_rng(62)
    h = cluster_rows(rng, 4, 32768, 64).astype(np.float32)
    widths = (16384, 16384)
    g, A = _stream(ops, h, 0.5, torch.float32, widths)
    for s_ in range(4):
        g1, A1 = _stream(ops, h[s_:s_ + 1], 0.5, torch.float32, widths)
        assert np.array_equal(g[s_], g1[0]), s_
        assert np.array_equal(A[s_], A1[0]), s_


# ------------------------------------------------------------------ streaming chunker

def _stream(ops, h, eps2, dtype, widths, inplace=False):
    """h [nseq, T, d] through windows of the given widths on the GPU, the
    carried matrix passed from window to window (updated in place if asked).
    Returns (dR [nseq, T], final carried matrix)."""
    nseq, T, d = h.shape
    assert sum(widths) == T
    out = np.empty((nseq, T), np.float32)
    state = None
    t = 0
    for w in widths:
        say("stream window", t, "+", w, "d", d, "inplace", inplace)
        win = to_dev(np.ascontiguousarray(h[:, t:t + w]), dtype)
        so = state if (inplace and state is not None) else None
        dR, state, st = ops.coding_rate_stream(win, eps2, state, state_out=so)
        assert int(to_np(st)[0]) == 0
        out[:, t:t + w] = to_np(dR)
        t += w
    return out, to_np(state)


def _oracle_stream(h, eps2, widths):
    outs, A, t = [], None, 0
    for w in widths:
        dr, A = oracle.coding_rate_stream(h[:, t:t + w].astype(np.float64), eps2, A)
        outs.append(dr)
        t += w
    return np.concatenate(outs, axis=1), A


@pytest.mark.parametrize("dt,d,widths,inplace", [
    ("f32", 40, (129, 1, 64, 70), False),
    ("f32", 64, (300, 256, 145), True),
    ("bf16", 128, (257, 3, 300), True),
    ("bf16", 72, (1, 130), False),
])
def test_coding_rate_stream_vs_oracle(ops, dt, d, widths, inplace):
    """Windows of ragged widths (a one-row window, widths off the block size,
    d off the 64-wide tiles) against the oracle's streaming chunker: every
    Delta R and the carried matrix after the last window."""
    torch = _torch()
    rng = np.random.default_rng(40 + d)
    h = cluster_rows(rng, 2, sum(widths), d)
    h = bf16_round(h) if dt == "bf16" else h.astype(np.float32)
    g, A = _stream(ops, h, 0.5, torch.bfloat16 if dt == "bf16" else torch.float32, widths, inplace)
    o, oA = _oracle_stream(h, 0.5, widths)
    assert np.max(np.abs(g - o) / np.abs(o)) < 1e-3
    assert np.max(np.abs(A - oA)) <= 1e-5 * np.max(np.abs(oA))
    assert np.array_equal(A, np.transpose(A, (0, 2, 1)))


def test_coding_rate_stream_state_out_optional(ops):
    """state_out NULL: Delta R of a later window is still exact, and the
    carried matrix passed in is left as it was."""
    torch = _torch()
    rng = np.random.default_rng(44)
    h = cluster_rows(rng, 1, 200, 64).astype(np.float32)
    _, A1 = oracle.coding_rate_stream(h[:, :120].astype(np.float64), 0.5)
    st_in = to_dev(A1.astype(np.float32))
    dR, none, st = ops.coding_rate_stream(to_dev(h[:, 120:], torch.float32), 0.5, st_in, want_state=False)
    assert none is None
    o, _ = oracle.coding_rate_stream(h[:, 120:].astype(np.float64), 0.5, A1.astype(np.float32))
    assert int(to_np(st)[0]) == 0
    assert np.max(np.abs(to_np(dR) - o) / np.abs(o)) < 1e-3
    assert np.array_equal(to_np(st_in), A1.astype(np.float32))


def test_topk_window_first_and_later_bitexact(ops):
    rng = np.random.default_rng(45)
    for W in (1, 2, 5, 1023, 1025, 3000):
        sc = rng.integers(0, 5, size=(2, W)).astype(np.float32)
        sc[0, ::9] = -0.0
        sc[1, ::5] = -np.inf
        for K in sorted({1, min(W, 2), max(1, W // 4), W}):
            for first in (True, False):
                idx, mask, _ = ops.topk_select_window(to_dev(sc), K, first)
                want = oracle.topk_select_window(sc, K, first)
                assert np.array_equal(to_np(idx), want), (W, K, first)
                assert np.array_equal(to_np(mask), oracle.topk_mask(want, W))
    sc = rng.standard_normal((1, 64)).astype(np.float32)
    sc[0, 0] = np.nan
    idx, _, st = ops.topk_select_window(to_dev(sc), 10, False)
    assert np.array_equal(to_np(idx), oracle.topk_select_window(sc, 10, False))
    assert 0 not in set(to_np(idx)[0].tolist()) and int(to_np(st)[0]) & 2


def test_streaming_chunker_full_size_bf16_32x8192x512_windows_1024(ops):
    """The 32 x 8192 x 512 bf16 workload streamed in windows of 1024 bytes
    with the carried matrix updated in place: sampled Delta R against the
    oracle's whole-sequence values (equal to the streamed ones by the
    oracle's own pin), window edges included; the streamed values against
    the whole-sequence kernel; the local Top-256 of every window equal to
    the oracle's selection on the device scores; the final carried matrix
    of one sequence against I + alpha H^T H in fp64."""
    torch = _torch()
    c = gen_byteflow_layer()
    W, Kw = 1024, 256
    g, A = _stream(ops, c["h"], c["eps2"], torch.bfloat16, (W,) * (c["T"] // W), inplace=True)
    rng = np.random.default_rng(46)
    for s in (0, 13, 31):
        pos = np.sort(np.concatenate([[1023, 1024, 4096, 8191], rng.choice(c["T"], 4, replace=False)]))
        o = oracle.coding_rate_at(c["h"][s], c["eps2"], pos)
        assert np.max(np.abs(g[s, pos] - o) / np.abs(o)) < 1e-3, s
    whole, st = _dr(ops, c["h"], c["eps2"], torch.bfloat16)
    assert st == 0
    assert np.max(np.abs(g - whole) / np.abs(whole)) < 1e-3
    for wi in range(c["T"] // W):
        sc = np.ascontiguousarray(g[:, wi * W:(wi + 1) * W])
        idx, _, _ = ops.topk_select_window(to_dev(sc), Kw, wi == 0)
        assert np.array_equal(to_np(idx), oracle.topk_select_window(sc, Kw, wi == 0)), wi
    h0 = c["h"][5].astype(np.float64)
    d = h0.shape[1]
    want = np.eye(d) + oracle.alpha_of(d, c["eps2"]) * h0.T @ h0
    assert np.max(np.abs(A[5] - want)) <= 1e-5 * np.max(np.abs(want))


# ------------------------------------------------------------------ gather + upsample

def test_gather_via_compact_on_topk_mask(ops):
    torch = _torch()
    rng = np.random.default_rng(11)
    nseq, T, d, K = 3, 1000, 64, 100
    h = bf16_round(rng.standard_normal((nseq, T, d)))
    sc = rng.standard_normal((nseq, T)).astype(np.float32)
    idx, mask, _ = ops.topk_select(to_dev(sc), K)
    off = np.arange(nseq + 1, dtype=np.int64) * T
    gi, coff, z, _, _ = ops.compact(mask.reshape(-1), to_dev(off), rows=to_dev(h.reshape(-1, d), torch.bfloat16))
    want = (to_np(idx) + off[:-1, None]).reshape(-1)
    assert np.array_equal(to_np(gi)[:nseq * K], want)
    assert np.array_equal(to_np(coff), np.arange(nseq + 1) * K)
    assert np.array_equal(to_np(z)[:nseq * K], oracle.gather(h, to_np(idx)).reshape(-1, d))


@pytest.mark.parametrize("dt,nseq,T,d,K", [("bf16", 3, 1000, 64, 100), ("f32", 2, 777, 8, 1), ("bf16", 2, 300, 512, 300),
                                          ("f32", 5, 4096, 200, 1025), ("bf16", 1, 4096, 4096, 33)])
def test_gather_topk_bitexact(ops, dt, nseq, T, d, K):
    """z = h at the Top-K positions, row for row, against the oracle's gather
    (K = 1, K = T, rows of 16 bytes to 8 KB); the same rows as the
    compaction on the Top-K mask."""
    torch = _torch()
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    rng = np.random.default_rng(nseq * 1000 + K)
    h = rng.standard_normal((nseq, T, d)).astype(np.float32)
    if dt == "bf16":
        h = bf16_round(h)
    sc = rng.standard_normal((nseq, T)).astype(np.float32)
    idx, mask, _ = ops.topk_select(to_dev(sc), K)
    hd = to_dev(h, tdt)
    z = ops.gather_topk(hd, idx)
    want = oracle.gather(h, to_np(idx))
    assert np.array_equal(to_np(z.float()), want.astype(np.float32))
    if nseq * T <= 20000:
        off = np.arange(nseq + 1, dtype=np.int64) * T
        _, _, zc, _, _ = ops.compact(mask.reshape(-1), to_dev(off), rows=hd.view(-1, d))
        assert torch.equal(zc[:nseq * K].view(nseq, K, d), z)


def test_gather_topk_clamps_indices(ops):
    """Positions outside [0, T) read the nearest row of the sequence; the
    library never reads outside h."""
    torch = _torch()
    h = np.arange(2 * 10 * 4, dtype=np.float32).reshape(2, 10, 4)
    idx = np.array([[-5, 0, 9, 10], [3, 12, -1, 7]], np.int32)
    z = ops.gather_topk(to_dev(h), to_dev(idx))
    want = oracle.gather(h, np.clip(idx, 0, 9))
    assert np.array_equal(to_np(z), want)


def _random_idx(rng, nseq, T, K):
    return np.stack([np.sort(np.concatenate([[0], rng.choice(np.arange(1, T), K - 1, replace=False)]))
                     for _ in range(nseq)]).astype(np.int32)


@pytest.mark.parametrize("nseq,T,K,dg,dl,B", [(3, 1000, 37, 96, 136, 4), (4, 3000, 300, 200, 320, 16)])
def test_upsample_plan_then_apply_equals_one_call(ops, nseq, T, K, dg, dl, B):
    """The plan on a second stream (ordered before the apply by an event),
    then the apply, gives bit for bit the one-call result; a second plan into
    the same workspace (other chunk starts) replaces the first."""
    torch = _torch()
    rng = np.random.default_rng(nseq * T + K)
    bf = torch.bfloat16
    g = to_dev(bf16_round(rng.standard_normal((nseq, K, dg))), bf)
    W = to_dev(bf16_round(rng.standard_normal((B, dg, dl)) / np.sqrt(dg)), bf)
    h = to_dev(bf16_round(rng.standard_normal((nseq, T, dl))), bf)
    ws = None
    for rep in range(2):
        idx = to_dev(_random_idx(rng, nseq, T, K))
        want = ops.upsample_bins(g, W, idx, h, B)
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            ws = ops.upsample_plan(idx, T, B, ws=ws)
            done = torch.cuda.Event()
            done.record(s2)
        torch.cuda.current_stream().wait_event(done)
        got = ops.upsample_apply(g, W, h, B, ws)
        assert torch.equal(got, want), rep


def test_upsample_positions_not_ascending_stay_in_bounds(ops):
    """Positions that are not ascending or fall outside [0, T) (here chunks
    that overlap, so their items outgrow the workspace's slots, and values
    far outside the sequence) are clamped: the call succeeds and writes
    nothing outside s_out (guard rows on both sides keep their contents)."""
    torch = _torch()
    rng = np.random.default_rng(5)
    nseq, T, K, dg, dl, B = 5, 500, 400, 64, 32, 16
    idx = _random_idx(rng, nseq, T, K)
    idx[1] = np.where(np.arange(K) % 2 == 0, 0, T)  # [0, T, 0, T, ...]: 200 chunks of length T
    idx[2] = idx[1]
    idx[3] = np.where(np.arange(K) % 2 == 0, -50, T + 50)
    idx[1, 7], idx[1, 9] = -7, 10 ** 6
    idx[4] = rng.integers(-100, T + 100, K)
    bf = torch.bfloat16
    g = to_dev(bf16_round(rng.standard_normal((nseq, K, dg))), bf)
    W = to_dev(bf16_round(rng.standard_normal((B, dg, dl)) / np.sqrt(dg)), bf)
    h = to_dev(bf16_round(rng.standard_normal((nseq, T, dl))), bf)
    G = 4096  # guard elements on each side (a multiple of 8: s_out stays 16-byte aligned)
    n = nseq * T * dl
    big = torch.full((n + 2 * G,), 7.0, dtype=bf, device="cuda")
    s = big[G:G + n].view(nseq, T, dl)
    ops.upsample_bins(g, W, to_dev(idx), h, B, s_out=s)
    torch.cuda.synchronize()
    assert bool((big[:G] == 7.0).all()) and bool((big[G + n:] == 7.0).all())


@pytest.mark.parametrize("nseq,T,K,dg,dl,B", [(2, 300, 40, 64, 32, 16), (3, 1000, 37, 96, 136, 4),
                                              (1, 64, 64, 32, 8, 16), (2, 500, 1, 64, 64, 16),
                                              (4, 3000, 300, 200, 320, 16), (2, 2000, 20, 64, 64, 64)])
def test_upsample_vs_oracle(ops, nseq, T, K, dg, dl, B):
    torch = _torch()
    rng = np.random.default_rng(T + K)
    idx = _random_idx(rng, nseq, T, K)
    g = bf16_round(rng.standard_normal((nseq, K, dg)))
    W = bf16_round(rng.standard_normal((B, dg, dl)) / np.sqrt(dg))
    h = bf16_round(rng.standard_normal((nseq, T, dl)))
    bf = torch.bfloat16
    s = ops.upsample_bins(to_dev(g, bf), to_dev(W, bf), to_dev(idx), to_dev(h, bf), B)
    ref = oracle.upsample_bins(g, W, idx, h, B)
    assert row_rel_err(to_np(s), ref) < 2e-2


def test_byteflow_chain_full_size_bf16_32x8192(ops):
    """32 x 8192 x 512 bf16 at full size (the launch configuration of bench.py): Delta R, Top-K,
    gather, global stand-in, 16-bin upsample + residual; every upsample row of
    four sequences checked against the oracle."""
    torch = _torch()
    bf = torch.bfloat16
    c = gen_byteflow_layer()
    nseq, T, K = c["nseq"], c["T"], c["K"]
    h_t = to_dev(c["h"], bf)
    dR, st = ops.coding_rate(h_t, c["eps2"])
    idx, mask, _ = ops.topk_select(dR, K)
    off = np.arange(nseq + 1, dtype=np.int64) * T
    gi, coff, z, _, _ = ops.compact(mask.reshape(-1), to_dev(off), rows=h_t.reshape(-1, c["d_local"]),
                                    capacity=nseq * K)
    z_np = to_np(z).reshape(nseq, K, -1)
    idx_np = to_np(idx)
    assert np.array_equal(z_np, oracle.gather(c["h"], idx_np))
    g = gen_global_standin(z_np, c)
    s = ops.upsample_bins(to_dev(g, bf), to_dev(c["w_bin"], bf), idx, h_t, c["nbins"])
    s_np = to_np(s)
    for q in (0, 10, 21, 31):
        ref = oracle.upsample_bins(g[q:q + 1], c["w_bin"], idx_np[q:q + 1], c["h"][q:q + 1], c["nbins"])
        err = row_rel_err(s_np[q:q + 1], ref)
        say("upsample seq", q, "max row rel err", err)
        assert err < 2e-2
    say("ByteFlow chain ok")


# ------------------------------------------------------------------ cosine-score chunker

def test_cosine_score_chunker_byteflow_shape(ops):
    """The cosine-similarity chunker variant: the H-Net routing score p_t of
    the encoder output, q = h Wq and k = h Wk, takes Delta R's place in the
    BOS + Top-(K-1) selection.  Four full sequences of the ByteFlow layer
    input (8192 x 512, K 2048)."""
    torch = _torch()
    bf = torch.bfloat16
    c = gen_byteflow_layer()
    nseq, T, K = 4, c["T"], c["K"]
    h = c["h"][:nseq]
    q, k = gen_cosine_qk(h, c)
    off = np.arange(nseq + 1, dtype=np.int64) * T
    p, _, _ = ops.route(to_dev(q, bf), to_dev(k, bf), to_dev(off), threshold=0.5)
    p_g = to_np(p).reshape(nseq, T)
    p_o = oracle.route(q, k, off).reshape(nseq, T)
    assert np.max(np.abs(p_g - p_o)) < 5e-6
    assert np.all(p_g[:, 0] == 1.0)
    idx, mask, st = ops.topk_select(p.reshape(nseq, T), K)
    idx_g = to_np(idx)
    # bit-exact on the device scores ...
    assert np.array_equal(idx_g, oracle.topk_select(p_g, K))
    assert np.array_equal(to_np(mask), oracle.topk_mask(idx_g, T))
    # ... and the oracle's own selection outside the tie band
    sel_o = oracle.topk_select(p_o.astype(np.float64), K)
    for s_ in range(nseq):
        diff, band = topk_band_compare(idx_g[s_], sel_o[s_], p_o[s_], K)
        assert len(diff) == 0, (s_, diff[:10], band)
    say("cosine chunker: selections agree")
