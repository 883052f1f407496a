"""Pins for the H-Net half of the oracle (route, quantile, compact, EMA dechunk)."""
import json
import os

import numpy as np
import pytest
from scipy.spatial.distance import cosine as scipy_cosine_distance

import oracle
from synthdata import gen_hnet_tiny, gen_event_streams

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_route_golden_hand_derived():
    g = _gold("hnet_tiny.json")
    p = oracle.route(np.array(g["q"]), np.array(g["k"]), np.array(g["offsets"]))
    np.testing.assert_allclose(p, g["p_expected"], atol=1e-12)


def test_route_matches_scipy_cosine_distance():
    c = gen_hnet_tiny()
    p = oracle.route(c["q"], c["k"], c["offsets"])
    off = c["offsets"]
    for s in range(len(off) - 1):
        assert p[off[s]] == 1.0
        for t in range(off[s] + 1, off[s + 1], 7):
            want = 0.5 * scipy_cosine_distance(c["q"][t].astype(np.float64), c["k"][t - 1].astype(np.float64))
            assert abs(p[t] - want) < 1e-12


def test_route_starts_and_range_ragged():
    c = gen_event_streams(nseq=4, d=64, min_events=2, max_events=6)
    p = oracle.route(c["q"], c["k"], c["offsets"])
    assert np.all(p[c["offsets"][:-1]] == 1.0)
    assert np.all((p >= 0) & (p <= 1))


def test_route_zero_row_gives_half():
    q = np.zeros((3, 4)); k = np.zeros((3, 4)); q[1] = 1.0
    p = oracle.route(q, k, np.array([0, 3]))
    assert p[1] == 0.5 and p[2] == 0.5


def test_quantile_matches_numpy_lower():
    rng = np.random.default_rng(3)
    for n in (1, 2, 7, 1000, 4097):
        p = rng.random(n)
        assert oracle.stage_quantile(p, 0.75) == np.quantile(p, 0.75, method="lower")


def test_quantile_keeps_about_a_quarter():
    c = gen_hnet_tiny(nseq=4, T=512)
    p = oracle.route(c["q"], c["k"], c["offsets"])
    tau = oracle.stage_quantile(p, 0.75)
    b = oracle.boundary_mask(p, tau)
    assert abs(b.mean() - 0.25) < 0.01


def test_boundary_mask_fp32_decision_and_nan():
    p = np.array([0.5, np.nextafter(0.5, 0), 0.7, np.nan])
    b = oracle.boundary_mask(p, 0.5)
    # nextafter(0.5, 0) in fp64 rounds to 0.5 in fp32: the decision is taken in fp32
    assert list(b) == [True, True, True, False]


def test_compact_scatter_recovers_rows_and_counts():
    c = gen_event_streams(nseq=5, d=32, min_events=2, max_events=9)
    p = oracle.route(c["q"], c["k"], c["offsets"])
    b = oracle.boundary_mask(p, 0.5)
    idx, coff, z, P = oracle.compact(b, p, c["h"], c["offsets"])
    assert len(idx) == int(b.sum()) == len(z) == len(P)
    back = np.zeros_like(c["h"])
    back[idx] = z
    assert np.array_equal(back[b], c["h"][b])
    assert np.array_equal(np.asarray(P), p[b])
    # chunk offsets by brute force per sequence
    off = c["offsets"]
    for s in range(len(off) - 1):
        assert coff[s + 1] - coff[s] == sum(1 for t in range(off[s], off[s + 1]) if b[t])
        assert idx[coff[s]] == off[s]  # every start is a boundary (p = 1)
    assert np.all(np.diff(idx) > 0)


def test_ema_golden_hand_derived():
    g = _gold("hnet_tiny.json")
    out = oracle.dechunk_ema(np.array(g["z"]), np.array(g["P"]), np.array(g["idx"]),
                             np.array([0, 3]), np.array(g["ema_offsets"]))
    np.testing.assert_allclose(out, g["ema_expected"], atol=1e-15)


def _ragged_chunks(rng, lengths, d, first_p_one=True):
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = offsets[-1]
    b = rng.random(N) < 0.4
    b[offsets[:-1]] = True
    p = rng.random(N)
    if first_p_one:
        p[offsets[:-1]] = 1.0
    rows = rng.standard_normal((N, d))
    idx, coff, z, P = oracle.compact(b, p, rows, offsets)
    return offsets, b, p, rows, idx, coff, z, P


def test_ema_identity_when_every_byte_is_a_boundary_with_P1():
    rng = np.random.default_rng(5)
    offsets = np.array([0, 7, 20, 21])
    rows = rng.standard_normal((21, 6)).astype(np.float32)
    b = np.ones(21, bool); p = np.ones(21)
    idx, coff, z, P = oracle.compact(b, p, rows, offsets)
    out = oracle.dechunk_ema(z, P, idx, coff, offsets)
    assert np.array_equal(out, rows.astype(np.float64))


def test_ema_constant_z_is_fixed_point():
    rng = np.random.default_rng(6)
    offsets, b, p, rows, idx, coff, z, P = _ragged_chunks(rng, [30, 11, 50], 5)
    v = rng.standard_normal(5)
    out = oracle.dechunk_ema(np.tile(v, (len(z), 1)), P, idx, coff, offsets)
    np.testing.assert_allclose(out, np.tile(v, (len(out), 1)), rtol=1e-14, atol=1e-14)


def test_ema_constant_P_geometric_closed_form():
    rng = np.random.default_rng(7)
    M, d, a = 40, 3, 0.3
    z = rng.standard_normal((M, d))
    P = np.full(M, a); P[0] = 1.0
    idx = np.arange(M); offsets = np.array([0, M]); coff = np.array([0, M])
    out = oracle.dechunk_ema(z, P, idx, coff, offsets)
    for c in range(M):
        want = (1 - a) ** c * z[0] + sum(a * (1 - a) ** (c - j) * z[j] for j in range(1, c + 1))
        np.testing.assert_allclose(out[c], want, rtol=1e-12, atol=1e-12)


def test_ema_stays_in_convex_hull_and_is_linear():
    rng = np.random.default_rng(8)
    offsets, b, p, rows, idx, coff, z, P = _ragged_chunks(rng, [64, 9, 33], 4)
    out = oracle.dechunk_ema(z, P, idx, coff, offsets)
    for s in range(3):
        for c in range(coff[s], coff[s + 1]):
            lo = z[coff[s]:c + 1].min(0) - 1e-12
            hi = z[coff[s]:c + 1].max(0) + 1e-12
            assert np.all(out[idx[c]] >= lo) and np.all(out[idx[c]] <= hi)
    z2 = rng.standard_normal(z.shape)
    lin = oracle.dechunk_ema(2.0 * z - 3.0 * z2, P, idx, coff, offsets)
    np.testing.assert_allclose(lin, 2.0 * out - 3.0 * oracle.dechunk_ema(z2, P, idx, coff, offsets), atol=1e-12)


def test_ema_chunk_form_equals_per_byte_form():
    """Per-byte scan zbar_t = P_t x_t + (1-P_t) zbar_{t-1} with P_t = p_t b_t
    (zbar reset to 0 at a start) gives the same result as the chunk scan."""
    rng = np.random.default_rng(9)
    offsets, b, p, rows, idx, coff, z, P = _ragged_chunks(rng, [25, 40, 3], 6, first_p_one=False)
    out = oracle.dechunk_ema(z, P, idx, coff, offsets)
    ref = np.zeros_like(out)
    for s in range(3):
        zb = np.zeros(6)
        for t in range(offsets[s], offsets[s + 1]):
            Pt = p[t] * b[t]
            zb = Pt * rows[t] + (1 - Pt) * zb if b[t] else zb
            ref[t] = zb
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- EMA backward

def _loss(z, P, idx, coff, offsets, dout):
    return float(np.sum(dout * oracle.dechunk_ema(z, P, idx, coff, offsets)))


def test_ema_backward_matches_central_differences():
    """dz and dP against central differences of the (pinned) forward, on a
    ragged batch with an empty sequence, a sequence whose first byte is not a
    boundary and P below 1 at sequence starts; the loss is linear in z, so its
    z-differences are exact up to rounding, and the quadratic terms in P
    cancel in central differences."""
    rng = np.random.default_rng(21)
    offsets = np.array([0, 9, 9, 23, 29], np.int64)
    N = int(offsets[-1])
    b = rng.random(N) < 0.4
    b[[0, 9, 23]] = True
    b[23:26] = False  # the last sequence starts without a boundary
    b[26] = True
    p = rng.random(N)
    idx, coff, z, P = oracle.compact(b, p, rng.standard_normal((N, 3)), offsets)
    dout = rng.standard_normal((N, 3))
    dz, dP = oracle.dechunk_ema_backward(z, P, idx, coff, offsets, dout)
    eps = 1e-6
    for c in range(len(P)):
        for f in range(3):
            zp, zm = z.copy(), z.copy()
            zp[c, f] += eps
            zm[c, f] -= eps
            fd = (_loss(zp, P, idx, coff, offsets, dout) - _loss(zm, P, idx, coff, offsets, dout)) / (2 * eps)
            assert abs(fd - dz[c, f]) <= 1e-7 * max(1.0, abs(fd))
        Pp, Pm = P.astype(np.float64).copy(), P.astype(np.float64).copy()
        Pp[c] += eps
        Pm[c] -= eps
        fd = (_loss(z, Pp, idx, coff, offsets, dout) - _loss(z, Pm, idx, coff, offsets, dout)) / (2 * eps)
        assert abs(fd - dP[c]) <= 1e-6 * max(1.0, abs(fd))


def test_ema_backward_P_one_closed_form():
    """With every P = 1 the output is each chunk's own z: dz_c is the sum of
    dout over the chunk's positions and dP_c = that sum . (z_c - z_{c-1}),
    with z_{c-1} = 0 at a sequence's first chunk."""
    rng = np.random.default_rng(22)
    offsets, b, p, rows, idx, coff, z, P = _ragged_chunks(rng, [12, 7, 30], 4)
    P1 = np.ones_like(P)
    dout = rng.standard_normal((int(offsets[-1]), 4))
    dz, dP = oracle.dechunk_ema_backward(z, P1, idx, coff, offsets, dout)
    for s in range(3):
        for c in range(coff[s], coff[s + 1]):
            t_end = idx[c + 1] if c + 1 < coff[s + 1] else offsets[s + 1]
            g = dout[idx[c]:t_end].sum(axis=0)
            prev = z[c - 1] if c > coff[s] else np.zeros(4)
            np.testing.assert_allclose(dz[c], g, rtol=1e-13, atol=1e-13)
            assert abs(dP[c] - g @ (z[c] - prev)) <= 1e-12 * max(1.0, abs(dP[c]))


def test_ema_backward_linear_in_dout():
    rng = np.random.default_rng(23)
    offsets, b, p, rows, idx, coff, z, P = _ragged_chunks(rng, [20, 11], 5, first_p_one=False)
    N = int(offsets[-1])
    g1, g2 = rng.standard_normal((N, 5)), rng.standard_normal((N, 5))
    a1 = oracle.dechunk_ema_backward(z, P, idx, coff, offsets, g1)
    a2 = oracle.dechunk_ema_backward(z, P, idx, coff, offsets, g2)
    a3 = oracle.dechunk_ema_backward(z, P, idx, coff, offsets, 2.0 * g1 - 3.0 * g2)
    np.testing.assert_allclose(a3[0], 2.0 * a1[0] - 3.0 * a2[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a3[1], 2.0 * a1[1] - 3.0 * a2[1], rtol=1e-12, atol=1e-12)
