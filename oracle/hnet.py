"""H-Net dynamic chunking, oracle side (fp64, plain loops).  Test infrastructure.

Follows [BG] section 2.3: the boundary probability comes from the cosine
similarity of adjacent byte representations, chosen boundaries are kept
(compaction into a shorter ragged sequence) and the coarse result is brought
back to byte length by an exponential moving average over chunks.
"""
from __future__ import annotations

import numpy as np


def route(q, k, offsets) -> np.ndarray:
    """Boundary probability per position, float64.

    p_t = (1 - cos(q_t, k_{t-1})) / 2 within a sequence, p = 1 at every
    sequence start (no pair crosses a sequence boundary).  cos = dot /
    max(|q||k|, 1e-12) so that a zero row gives cos = 0; p is clamped to [0,1].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n = q.shape[0]
    p = np.empty(n, dtype=np.float64)
    for s in range(len(offsets) - 1):
        a, b = int(offsets[s]), int(offsets[s + 1])
        if b <= a:
            continue
        p[a] = 1.0
        for t in range(a + 1, b):
            qt, kp = q[t], k[t - 1]
            den = max(np.sqrt(qt @ qt) * np.sqrt(kp @ kp), 1e-12)
            cos = (qt @ kp) / den
            p[t] = min(max(0.5 * (1.0 - cos), 0.0), 1.0)
    return p


def boundary_mask(p, tau) -> np.ndarray:
    """b_t = [p_t >= tau], decided in fp32 (the precision the kernel decides in):
    both p and tau are rounded to float32 first.  NaN p gives no boundary."""
    return (np.asarray(p, dtype=np.float32) >= np.float32(tau))


def stage_quantile(p, quantile: float) -> float:
    """Stage threshold: the lower ``quantile`` order statistic of all valid
    positions' scores, v[floor(quantile * (n-1))] of the ascending sort.
    With quantile 0.75 about a quarter of the positions are kept per stage
    ([BG] 2.3: stages at 1/4 and 1/16 of the original length)."""
    v = np.sort(np.asarray(p, dtype=np.float64))
    n = len(v)
    r = int(np.floor(quantile * (n - 1)))
    return float(v[r])


def compact(b, p, rows, offsets):
    """Keep boundary positions.  Returns (idx, chunk_offsets, z, P):
    idx = global positions with b = 1 in increasing order, chunk_offsets[s] =
    number of boundaries before sequence s starts, z = rows[idx], P = p[idx]."""
    b = np.asarray(b).astype(bool)
    idx = np.flatnonzero(b)
    before = np.concatenate([[0], np.cumsum(b)])
    chunk_offsets = before[np.asarray(offsets, dtype=np.int64)].astype(np.int64)
    z = None if rows is None else np.asarray(rows)[idx]
    P = None if p is None else np.asarray(p)[idx]
    return idx.astype(np.int64), chunk_offsets, z, P


def dechunk_ema(z, P, idx, chunk_offsets, offsets) -> np.ndarray:
    """EMA dechunk back to byte length, float64 [N x d].

    Per sequence, over its chunks c in order:
        zbar_c = P_c * z_c + (1 - P_c) * zbar_{c-1},   zbar before the first chunk = 0,
    and every position t of the sequence takes zbar of the chunk holding it
    (the last chunk starting at or before t).  Positions before a
    sequence's first boundary (impossible when starts are boundaries) get 0.
    """
    z = np.asarray(z, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    N = int(offsets[-1])
    out = np.zeros((N, z.shape[1]), dtype=np.float64)
    for s in range(len(offsets) - 1):
        c0, c1 = int(chunk_offsets[s]), int(chunk_offsets[s + 1])
        zbar = np.zeros(z.shape[1])
        for c in range(c0, c1):
            zbar = P[c] * z[c] + (1.0 - P[c]) * zbar
            t_end = int(idx[c + 1]) if c + 1 < c1 else int(offsets[s + 1])
            out[int(idx[c]):t_end] = zbar
    return out


def dechunk_ema_backward(z, P, idx, chunk_offsets, offsets, dout):
    """Gradients of L = sum(dout * dechunk_ema(z, P, ...)) with respect to z
    and P, float64 ([M x d] and [M]).

    [BG] 2.3 smooths the chunk sequence with the EMA so that the boundary
    choice stays differentiable end to end; this is the reverse-mode
    derivative of that recurrence, taken chunk by chunk per sequence:
        gbar_c = sum of dout over the positions chunk c covers
        lam_c  = gbar_c + (1 - P_{c+1}) lam_{c+1}   (lam_c = gbar_c for the
                 sequence's last chunk: the next sequence restarts from 0)
        dz_c   = P_c lam_c
        dP_c   = lam_c . (z_c - zbar_{c-1})          (zbar before the first chunk = 0)
    lam_c is dL/dzbar_c; positions before a sequence's first chunk do not
    depend on z or P.
    """
    z = np.asarray(z, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    M, d = z.shape[0], z.shape[1]
    dz = np.zeros((M, d), dtype=np.float64)
    dP = np.zeros(M, dtype=np.float64)
    for s in range(len(offsets) - 1):
        c0, c1 = int(chunk_offsets[s]), int(chunk_offsets[s + 1])
        if c0 == c1:
            continue
        # forward values zbar_{c-1} seen by each chunk
        zprev = np.zeros((c1 - c0, d))
        zbar = np.zeros(d)
        for c in range(c0, c1):
            zprev[c - c0] = zbar
            zbar = P[c] * z[c] + (1.0 - P[c]) * zbar
        lam_next = np.zeros(d)
        for c in range(c1 - 1, c0 - 1, -1):
            t_end = int(idx[c + 1]) if c + 1 < c1 else int(offsets[s + 1])
            gbar = dout[int(idx[c]):t_end].sum(axis=0)
            lam = gbar + ((1.0 - P[c + 1]) * lam_next if c + 1 < c1 else 0.0)
            dz[c] = P[c] * lam
            dP[c] = float(np.dot(lam, z[c] - zprev[c - c0]))
            lam_next = lam
    return dz, dP
