"""ByteFlow coding-rate chunking and multi-linear upsampling, oracle side.
Test infrastructure (fp64, plain loops).

Coding rate ([BF4] prerequisites, lossy coding rate; [BF4] method, with
d = d_local):  R_eps(H) = 1/2 logdet(I_T + alpha H H^T), alpha = d / eps^2,
H in R^{T x d}.  By Sylvester's determinant identity this equals
1/2 logdet(I_d + alpha H^T H), which is what is evaluated here: the d x d
matrix of each prefix is factored afresh (Cholesky) and R = sum log diag(L).
Marginal rate ([BF4] stage 2):  Delta R_t = R(h_1..t) - R(h_1..t-1).
"""
from __future__ import annotations

import numpy as np


def alpha_of(d: int, eps2: float) -> float:
    """alpha = d / eps^2 with d = d_local ([BF4] method section).  No 1/T factor."""
    return float(d) / float(eps2)


def _rate(A) -> float:
    """1/2 logdet(A) for SPD A via Cholesky: sum of log of the factor's diagonal."""
    return float(np.sum(np.log(np.diag(np.linalg.cholesky(A)))))


def coding_rate(h, eps2: float) -> np.ndarray:
    """Delta R_t for every position of every sequence; h is [nseq, T, d] or [T, d].

    Position 0 (0-based) gets R(h_1) itself (R of the empty prefix is 0), so the
    values telescope to R(h_1..T); the pages start Delta R at the second
    position and always keep the first one as BOS, so this value never
    decides a boundary."""
    h = np.asarray(h, dtype=np.float64)
    squeeze = h.ndim == 2
    if squeeze:
        h = h[None]
    nseq, T, d = h.shape
    a = alpha_of(d, eps2)
    out = np.empty((nseq, T))
    for s in range(nseq):
        A = np.eye(d)
        r_prev = 0.0
        for t in range(T):
            A = A + a * np.outer(h[s, t], h[s, t])
            r = _rate(A)
            out[s, t] = r - r_prev
            r_prev = r
    return out[0] if squeeze else out


def coding_rate_at(h, eps2: float, positions) -> np.ndarray:
    """Delta R_t of one sequence h [T, d] at selected 0-based positions only
    (same definition as ``coding_rate``; the prefix matrices are rebuilt from
    running sums of outer products)."""
    h = np.asarray(h, dtype=np.float64)
    T, d = h.shape
    a = alpha_of(d, eps2)
    pos = np.asarray(positions, dtype=np.int64)
    need = sorted(set(int(t) for t in pos) | set(int(t) - 1 for t in pos if t > 0))
    rates = {-1: 0.0}
    G = np.zeros((d, d))
    cur = 0
    for t in need:
        while cur <= t:
            G += np.outer(h[cur], h[cur])
            cur += 1
        rates[t] = _rate(np.eye(d) + a * G)
    return np.array([rates[int(t)] - rates[int(t) - 1] for t in pos])


def topk_select(score, K: int) -> np.ndarray:
    """Boundary set S per sequence ([BF4] stage 2, [BF2] key design 2):
    position 0 (BOS) always, plus the K-1 largest scores among positions
    1..T-1, returned in increasing time order.  Ties are broken by the
    earlier position; NaN ranks below every number.  score: [nseq, T]."""
    score = np.asarray(score)
    squeeze = score.ndim == 1
    if squeeze:
        score = score[None]
    nseq, T = score.shape
    if not (1 <= K <= T):
        raise ValueError("need 1 <= K <= T")
    out = np.empty((nseq, K), dtype=np.int64)
    for s in range(nseq):
        cand = list(range(1, T))
        key = lambda t: (0 if np.isnan(score[s, t]) else 1, 0.0 if np.isnan(score[s, t]) else float(score[s, t]), -t)
        chosen = sorted(cand, key=key, reverse=True)[:K - 1]
        out[s] = sorted([0] + chosen)
    return out[0] if squeeze else out


def coding_rate_stream(h, eps2: float, A_in=None):
    """Delta R_t of one window of a byte stream, given the carried prefix matrix.

    The streaming chunker that the [BF4] weakness analysis suggests for
    autoregressive inference (sliding window with a local Top-K): the bytes
    arrive in windows, and the chunker carries A = I_d + alpha sum h h^T over
    every byte already seen.  Delta R is causal, so with that carry each
    window's values are the whole-sequence values (same definition as
    ``coding_rate``): A <- A + alpha h_t h_t^T, Delta R_t = R(A) - R(A before).
    h: [nseq, W, d] or [W, d]; A_in: [nseq, d, d] (or [d, d]), None for the
    stream's start (A = I).  Returns (dR [nseq, W], A_out [nseq, d, d])."""
    h = np.asarray(h, dtype=np.float64)
    squeeze = h.ndim == 2
    if squeeze:
        h = h[None]
    nseq, W, d = h.shape
    a = alpha_of(d, eps2)
    if A_in is None:
        A_in = np.broadcast_to(np.eye(d), (nseq, d, d))
    A_in = np.asarray(A_in, dtype=np.float64).reshape(nseq, d, d)
    out = np.empty((nseq, W))
    A_out = np.empty((nseq, d, d))
    for s in range(nseq):
        A = A_in[s].copy()
        r_prev = _rate(A)
        for t in range(W):
            A = A + a * np.outer(h[s, t], h[s, t])
            r = _rate(A)
            out[s, t] = r - r_prev
            r_prev = r
        A_out[s] = A
    if squeeze:
        return out[0], A_out[0]
    return out, A_out


def topk_select_window(score, K: int, first: bool) -> np.ndarray:
    """Local Top-K of one window of a stream.  The stream's first window is
    selected as a whole sequence (``topk_select``: BOS plus K-1); every later
    window keeps its K largest scores, with no forced position (the stream's
    BOS lies in the first window).  Ties go to the earlier position, NaN ranks
    below every number; the set is returned in time order (positions inside
    the window).  score: [nseq, W]."""
    if first:
        return topk_select(score, K)
    score = np.asarray(score)
    squeeze = score.ndim == 1
    if squeeze:
        score = score[None]
    nseq, W = score.shape
    if not (1 <= K <= W):
        raise ValueError("need 1 <= K <= W")
    out = np.empty((nseq, K), dtype=np.int64)
    for s in range(nseq):
        key = lambda t: (0 if np.isnan(score[s, t]) else 1, 0.0 if np.isnan(score[s, t]) else float(score[s, t]), -t)
        out[s] = sorted(sorted(range(W), key=key, reverse=True)[:K])
    return out[0] if squeeze else out


def topk_mask(idx, T: int) -> np.ndarray:
    idx = np.atleast_2d(idx)
    m = np.zeros((idx.shape[0], T), dtype=np.uint8)
    for s in range(idx.shape[0]):
        m[s, idx[s]] = 1
    return m


def gather(h, idx) -> np.ndarray:
    """z_1..K = [h_{s_1}, ..., h_{s_K}] per sequence ([BF4] stage 2, before W_proj)."""
    h = np.asarray(h)
    idx = np.atleast_2d(idx)
    return np.stack([h[s][idx[s]] for s in range(idx.shape[0])])


def chunk_bins(idx, T: int, nbins: int):
    """Chunk map and bin of every position of one sequence ([BF4] stage 4,
    [BF2] key design 4).  c(t) = the last i with s_i <= t.  The bin is the
    relative position inside the chunk: bin(t) = floor(nbins * (t - s_c) / L_c)
    with L_c = s_{c+1} - s_c (s_{K+1} = T), in exact integer arithmetic."""
    idx = np.asarray(idx, dtype=np.int64)
    c = np.empty(T, dtype=np.int64)
    bins = np.empty(T, dtype=np.int64)
    for i in range(len(idx)):
        s0 = int(idx[i])
        s1 = int(idx[i + 1]) if i + 1 < len(idx) else T
        L = s1 - s0
        for t in range(s0, s1):
            c[t] = i
            bins[t] = (nbins * (t - s0)) // L
    return c, bins


def upsample_bins(g, W, idx, h, nbins: int) -> np.ndarray:
    """Multi-linear reconstruction with the large residual ([BF4] stage 4,
    [BF2] key design 4):  s_t = h_t + g_{c(t)} W_{bin(t)}, row-vector
    convention, W_b in R^{d_global x d_local}.  g [nseq,K,dg], W [B,dg,dl],
    idx [nseq,K], h [nseq,T,dl]; returns float64 [nseq,T,dl]."""
    g = np.asarray(g, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    idx = np.atleast_2d(idx)
    nseq, T, dl = h.shape
    out = np.empty_like(h)
    for s in range(nseq):
        c, bins = chunk_bins(idx[s], T, nbins)
        for t in range(T):
            out[s, t] = h[s, t] + g[s, c[t]] @ W[bins[t]]
    return out
