"""Pins for the ByteFlow half of the oracle (coding rate, Top-K, gather, bins, upsample)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from synthdata import cluster_rows, gen_coding_rate_tiny

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- coding rate

def test_coding_rate_golden_hand_derived():
    g = _gold("coding_rate_tiny.json")
    dr = oracle.coding_rate(np.array(g["h"]), g["eps2"])
    np.testing.assert_allclose(dr, g["expected"], rtol=1e-12)


def test_coding_rate_brute_force_txt_form():
    """Against the pages' own T x T form: R(h_1..t) = 1/2 slogdet(I_t + alpha H H^T)."""
    c = gen_coding_rate_tiny()
    h = c["h"].astype(np.float64)
    a = c["d"] / c["eps2"]
    dr = oracle.coding_rate(h, c["eps2"])
    prev = 0.0
    for t in range(1, c["T"] + 1):
        H = h[:t]
        sign, ld = np.linalg.slogdet(np.eye(t) + a * H @ H.T)
        assert sign > 0
        assert abs(dr[t - 1] - (0.5 * ld - prev)) < 1e-10
        prev = 0.5 * ld


def test_coding_rate_telescopes():
    rng = np.random.default_rng(1)
    h = cluster_rows(rng, 1, 96, 16)[0]
    dr = oracle.coding_rate(h, 0.5)
    a = 16 / 0.5
    _, ld = np.linalg.slogdet(np.eye(96) + a * h @ h.T)
    assert abs(dr.sum() - 0.5 * ld) < 1e-9


def test_coding_rate_closed_forms():
    a_eps2 = 0.25
    d = 6
    a = d / a_eps2
    # orthogonal rows: each adds 1/2 log(1 + alpha |h|^2)
    Q, _ = np.linalg.qr(np.random.default_rng(2).standard_normal((d, d)))
    h = Q[:5] * np.array([[0.5], [1.0], [2.0], [0.1], [3.0]])
    dr = oracle.coding_rate(h, a_eps2)
    np.testing.assert_allclose(dr, 0.5 * np.log1p(a * (h ** 2).sum(1)), rtol=1e-12)
    # n repeats of a unit vector u: Delta R_n = 1/2 log((1 + alpha n) / (1 + alpha (n-1)))
    u = Q[0]
    dr = oracle.coding_rate(np.tile(u, (7, 1)), a_eps2)
    n = np.arange(1, 8)
    np.testing.assert_allclose(dr, 0.5 * np.log((1 + a * n) / (1 + a * (n - 1))), rtol=1e-11)


def test_coding_rate_invariances_and_bounds():
    rng = np.random.default_rng(3)
    h = cluster_rows(rng, 1, 40, 8)[0] * rng.uniform(0.5, 2.0, size=(40, 1))
    dr = oracle.coding_rate(h, 0.5)
    Q, _ = np.linalg.qr(rng.standard_normal((8, 8)))
    np.testing.assert_allclose(oracle.coding_rate(h @ Q, 0.5), dr, rtol=1e-10)
    np.testing.assert_allclose(oracle.coding_rate(3.0 * h, 0.5 * 9.0), dr, rtol=1e-10)
    a = 8 / 0.5
    n2 = (h ** 2).sum(1)
    before = np.concatenate([[0.0], np.cumsum(n2)[:-1]])
    lo = 0.5 * np.log1p(a * n2 / (1 + a * before))
    hi = 0.5 * np.log1p(a * n2)
    assert np.all(dr >= lo - 1e-12) and np.all(dr <= hi + 1e-12)


def test_coding_rate_at_matches_full_sweep():
    rng = np.random.default_rng(4)
    h = cluster_rows(rng, 1, 64, 8)[0]
    full = oracle.coding_rate(h, 0.5)
    pos = [0, 1, 5, 33, 63]
    np.testing.assert_allclose(oracle.coding_rate_at(h, 0.5, pos), full[pos], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- Top-K

def test_topk_golden_hand_derived():
    g = _gold("byteflow_tiny.json")
    assert list(oracle.topk_select(np.array(g["score"]), g["K"])) == g["topk_expected"]


def test_topk_matches_stable_argsort():
    rng = np.random.default_rng(5)
    sc = rng.random((3, 300)).astype(np.float32)
    sc[:, 50:60] = 0.5  # ties
    for K in (1, 2, 17, 100, 300):
        got = oracle.topk_select(sc, K)
        for s in range(3):
            order = np.argsort(-sc[s, 1:].astype(np.float64), kind="stable") + 1
            want = np.sort(np.concatenate([[0], order[:K - 1]]))
            assert np.array_equal(got[s], want)


def test_topk_brute_force_enumeration():
    rng = np.random.default_rng(6)
    for T in (2, 5, 9):
        sc = rng.integers(0, 4, size=T).astype(np.float64)  # many exact ties
        for K in range(1, T + 1):
            got = set(oracle.topk_select(sc, K).tolist())
            ok = []
            for sub in itertools.combinations(range(1, T), K - 1):
                S = set(sub)
                dom = all((sc[i] > sc[j]) or (sc[i] == sc[j] and i < j)
                          for i in S for j in range(1, T) if j not in S)
                if dom:
                    ok.append({0} | S)
            assert len(ok) == 1 and ok[0] == got


def test_topk_invariants_and_nan():
    rng = np.random.default_rng(7)
    sc = rng.standard_normal((2, 64))
    sc[1, 10] = np.nan
    idx = oracle.topk_select(sc, 20)
    for s in range(2):
        assert idx[s, 0] == 0 and len(idx[s]) == 20 and np.all(np.diff(idx[s]) > 0)
        chosen = set(idx[s, 1:].tolist())
        rest = [t for t in range(1, 64) if t not in chosen]
        assert min(np.nan_to_num(sc[s, list(chosen)], nan=-np.inf)) >= max(np.nan_to_num(sc[s, rest], nan=-np.inf))
    assert 10 not in set(idx[1].tolist())
    assert np.array_equal(oracle.topk_select(sc, 64)[0], np.arange(64))


# ---------------------------------------------------------------- streaming chunker

def test_coding_rate_stream_windows_equal_whole_sequence():
    """Windows of ragged widths with the carried matrix give the pinned
    whole-sequence values, and the final carry is I + alpha H^T H."""
    rng = np.random.default_rng(31)
    h = cluster_rows(rng, 2, 40, 8)
    eps2 = 0.7
    whole = oracle.coding_rate(h, eps2)
    A = None
    t = 0
    for w in (7, 1, 20, 12):
        dr, A = oracle.coding_rate_stream(h[:, t:t + w], eps2, A)
        np.testing.assert_allclose(dr, whole[:, t:t + w], rtol=1e-10, atol=1e-12)
        t += w
    a = 8 / eps2
    for s in range(2):
        np.testing.assert_allclose(A[s], np.eye(8) + a * h[s].T @ h[s], rtol=1e-13, atol=1e-12)


def test_coding_rate_stream_closed_forms_with_a_carry():
    """After one past row u: a row orthogonal to u adds 1/2 log(1 + alpha|v|^2);
    the row c u adds 1/2 log((1 + alpha (1 + c^2)|u|^2) / (1 + alpha|u|^2))."""
    d, eps2 = 5, 0.5
    a = d / eps2
    u = np.array([0.3, -0.2, 0.5, 0.0, 0.1])
    A_in = np.eye(d) + a * np.outer(u, u)
    v = np.array([0.2, 0.3, 0.0, 0.7, 0.0])
    assert abs(u @ v) < 1e-15
    c = 1.7
    dr, A_out = oracle.coding_rate_stream(np.stack([v]), eps2, A_in)
    assert abs(dr[0] - 0.5 * np.log1p(a * v @ v)) < 1e-13
    dr, _ = oracle.coding_rate_stream(np.stack([c * u]), eps2, A_in)
    uu = u @ u
    assert abs(dr[0] - 0.5 * np.log((1 + a * (1 + c * c) * uu) / (1 + a * uu))) < 1e-13
    # no carry: the stream's start is the whole-sequence definition
    dr0, _ = oracle.coding_rate_stream(np.stack([c * u]), eps2)
    assert abs(dr0[0] - 0.5 * np.log1p(a * c * c * uu)) < 1e-13


def test_topk_window_first_is_whole_sequence_rule():
    rng = np.random.default_rng(32)
    sc = rng.random((2, 50))
    for K in (1, 5, 50):
        assert np.array_equal(oracle.topk_select_window(sc, K, True), oracle.topk_select(sc, K))


def test_topk_window_later_brute_force_enumeration():
    """A later window keeps the unique K-subset whose every member beats every
    non-member (larger score, or equal and earlier); position 0 is not forced."""
    rng = np.random.default_rng(33)
    for W in (1, 4, 8):
        sc = rng.integers(0, 3, size=W).astype(np.float64)
        if W > 1:
            sc[0] = -1.0  # the lowest score, so a forced position 0 would show
        for K in range(1, W + 1):
            got = set(oracle.topk_select_window(sc, K, False).tolist())
            ok = []
            for sub in itertools.combinations(range(W), K):
                S = set(sub)
                if all((sc[i] > sc[j]) or (sc[i] == sc[j] and i < j) for i in S for j in range(W) if j not in S):
                    ok.append(S)
            assert len(ok) == 1 and ok[0] == got
    sc = np.array([0.5, np.nan, 0.1, 0.9])
    assert list(oracle.topk_select_window(sc, 3, False)) == [0, 2, 3]


# ---------------------------------------------------------------- gather / bins / upsample

def test_chunk_bins_golden_hand_derived():
    g = _gold("byteflow_tiny.json")
    c, b = oracle.chunk_bins(np.array(g["bins_idx"]), g["bins_T"], g["nbins"])
    assert list(c) == g["chunk_expected"] and list(b) == g["bins_expected"]


def test_chunk_bins_properties():
    rng = np.random.default_rng(8)
    T, B = 500, 16
    idx = np.sort(np.concatenate([[0], rng.choice(np.arange(1, T), 60, replace=False)]))
    c, b = oracle.chunk_bins(idx, T, B)
    assert np.all((b >= 0) & (b < B))
    for i in range(len(idx)):
        s0 = idx[i]; s1 = idx[i + 1] if i + 1 < len(idx) else T
        L = s1 - s0
        assert b[s0] == 0 and np.all(np.diff(b[s0:s1]) >= 0) and np.all(c[s0:s1] == i)
        if L >= B:
            assert set(b[s0:s1].tolist()) == set(range(B))
        if L % B == 0:
            assert np.all(np.bincount(b[s0:s1], minlength=B) == L // B)
    # every chunk of length exactly B: bin = t - s_c
    idx16 = np.arange(0, 160, 16)
    c, b = oracle.chunk_bins(idx16, 160, 16)
    assert np.array_equal(b, np.arange(160) - idx16[c])


def test_upsample_equal_bins_reduce_to_one_matmul_and_zero_g():
    rng = np.random.default_rng(9)
    nseq, T, K, dg, dl, B = 2, 40, 7, 12, 8, 4
    h = rng.standard_normal((nseq, T, dl))
    g = rng.standard_normal((nseq, K, dg))
    W1 = rng.standard_normal((dg, dl))
    W = np.tile(W1, (B, 1, 1))
    idx = np.stack([np.sort(np.concatenate([[0], rng.choice(np.arange(1, T), K - 1, replace=False)]))
                    for _ in range(nseq)])
    s = oracle.upsample_bins(g, W, idx, h, B)
    for q in range(nseq):
        c, _ = oracle.chunk_bins(idx[q], T, B)
        np.testing.assert_allclose(s[q], h[q] + (g[q] @ W1)[c], rtol=1e-12, atol=1e-12)
    W = rng.standard_normal((B, dg, dl))
    assert np.array_equal(oracle.upsample_bins(np.zeros_like(g), W, idx, h, B), h)


def test_upsample_uses_the_bin_of_each_position():
    """Bins picked one at a time: W_b = e_b-selector, so s - h reveals bin(t)."""
    rng = np.random.default_rng(10)
    T, B, K = 50, 4, 6
    idx = np.sort(np.concatenate([[0], rng.choice(np.arange(1, T), K - 1, replace=False)]))
    g = np.ones((1, K, 1))
    W = np.arange(1, B + 1, dtype=np.float64).reshape(B, 1, 1)  # W_b = b+1
    s = oracle.upsample_bins(g, W, idx[None], np.zeros((1, T, 1)), B)
    _, b = oracle.chunk_bins(idx, T, B)
    assert np.array_equal(s[0, :, 0], b + 1.0)


def test_gather_picks_rows_in_time_order():
    h = np.arange(2 * 10 * 3, dtype=np.float64).reshape(2, 10, 3)
    idx = np.array([[0, 4, 9], [0, 1, 2]])
    z = oracle.gather(h, idx)
    assert np.array_equal(z[0], h[0, [0, 4, 9]]) and np.array_equal(z[1], h[1, :3])


def test_topk_mask_hand_written():
    """The mask of a boundary set, written out by hand: 1 exactly at the
    selected positions, one row per sequence, uint8."""
    m = oracle.topk_mask([[0, 2, 5], [0, 1, 3]], 6)
    assert m.dtype == np.uint8
    assert np.array_equal(m, np.array([[1, 0, 1, 0, 0, 1], [1, 1, 0, 1, 0, 0]], np.uint8))
    one = oracle.topk_mask(np.array([0, 4]), 5)  # a single sequence given as one row
    assert np.array_equal(one, np.array([[1, 0, 0, 0, 1]], np.uint8))
    assert np.array_equal(oracle.topk_mask([[0, 1, 2]], 3), np.ones((1, 3), np.uint8))  # K = T
