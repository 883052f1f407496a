"""Shared test helpers: device transfer, tolerances, a parallel driver for the oracle."""
from __future__ import annotations

import multiprocessing as mp
import os
import sys

import numpy as np


def to_dev(x, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def row_rel_err(x, y):
    """max over rows of ||x - y||_2 / ||y||_2 (rows with ||y|| = 0 compare absolute)."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, np.shape(x)[-1])
    y = np.asarray(y, dtype=np.float64).reshape(-1, np.shape(y)[-1])
    num = np.linalg.norm(x - y, axis=1)
    den = np.linalg.norm(y, axis=1)
    return float(np.max(np.where(den > 0, num / np.maximum(den, 1e-300), num))) if len(x) else 0.0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dr_range(args):
    from threadpoolctl import threadpool_limits
    import oracle
    h, eps2, a, b = args
    with threadpool_limits(limits=1):  # one BLAS thread per worker process
        return oracle.coding_rate_at(h, eps2, np.arange(a, b))


def oracle_dr_parallel(h, eps2, nproc=None):
    """Delta R of one sequence h [T, d] from the oracle, position ranges spread
    over worker processes (each worker rebuilds its own prefix)."""
    T = h.shape[0]
    nproc = nproc or min(16, os.cpu_count() or 1)
    cuts = np.linspace(0, T, nproc + 1).astype(int)
    jobs = [(h, eps2, int(cuts[i]), int(cuts[i + 1])) for i in range(nproc) if cuts[i + 1] > cuts[i]]
    ctx = mp.get_context("fork")
    with ctx.Pool(len(jobs)) as pool:
        parts = pool.map(_dr_range, jobs)
    return np.concatenate(parts)


def topk_band_compare(sel_gpu, sel_or, dr_or, K, band=1e-5):
    """Compare two Top-K sets (one sequence) outside the band |dR - dR_(K)| <= band,
    where dR_(K) is the K-1-th largest oracle value among positions >= 1."""
    vK = np.sort(dr_or[1:])[::-1][K - 2] if K > 1 else np.inf
    T = len(dr_or)
    outside = np.abs(dr_or - vK) > band
    outside[0] = True
    a = np.zeros(T, bool); a[sel_gpu] = True
    b = np.zeros(T, bool); b[sel_or] = True
    return np.flatnonzero((a != b) & outside), int(np.sum(~outside))
