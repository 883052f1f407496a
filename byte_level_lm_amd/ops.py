"""Python binding of the chunk-layer C ABI (same names as include/bllm.h).

Argument marshalling only: each function checks shapes and dtypes, allocates
outputs/workspaces with torch when the caller does not pass them, and calls
the HIP library on torch's current stream.  Every step of the computation
runs in the library's kernels.  Nothing here synchronises: data-dependent
results (counts, status words) stay on the device until the caller reads them.
"""
from __future__ import annotations

import torch

from . import _lib as L


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return L.F32
    if t.dtype == torch.bfloat16:
        return L.BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ws(nbytes: int, ws, device):
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return ws
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _nbytes(t):
    return t.numel() * t.element_size()


# ------------------------------------------------------------------ sizes

def route_workspace(total: int) -> int:
    return int(L.lib().bllm_route_workspace(total))


def compact_workspace(total: int) -> int:
    return int(L.lib().bllm_compact_workspace(total))


def dechunk_workspace(d: int) -> int:
    return int(L.lib().bllm_dechunk_workspace(d))


def coding_rate_workspace(nseq: int, T: int, d: int) -> int:
    return int(L.lib().bllm_coding_rate_workspace(nseq, T, d))


def upsample_workspace(nseq: int, T: int, K: int, d_global: int, d_local: int, nbins: int) -> int:
    return int(L.lib().bllm_upsample_workspace(nseq, T, K, d_global, d_local, nbins))


# ------------------------------------------------------------------ ops

def route(q, k, offsets, *, threshold: float = 0.5, quantile=None, p_out=None, b_out=None,
          tau_out=None, status=None, ws=None):
    """H-Net boundary scores p, mask b and threshold tau (device tensors).
    `status` (int32 [1], device, optional) receives BLLM_S_INCOMPLETE if the
    quantile's bounded device-side wait gave up."""
    _dev(q, k, offsets)
    total, d = q.shape
    if k.shape != q.shape or k.dtype != q.dtype or offsets.dtype != torch.int64:
        raise ValueError("q and k must match; offsets must be int64")
    dev = q.device
    p_out = torch.empty(total, dtype=torch.float32, device=dev) if p_out is None else p_out
    b_out = torch.empty(total, dtype=torch.uint8, device=dev) if b_out is None else b_out
    tau_out = torch.empty(1, dtype=torch.float32, device=dev) if tau_out is None else tau_out
    quant = -1.0 if quantile is None else float(quantile)
    w = _ws(route_workspace(total), ws, dev) if quantile is not None else ws
    rc = L.lib().bllm_route(q.data_ptr(), k.data_ptr(), _dt(q), d, offsets.data_ptr(),
                            offsets.numel() - 1, total, float(threshold), quant, p_out.data_ptr(),
                            b_out.data_ptr(), tau_out.data_ptr(), _ptr(status), _ptr(w),
                            0 if w is None else _nbytes(w), _stream())
    L.check("bllm_route", rc)
    return p_out, b_out, tau_out


def route_fused(h, Wq, Wk, offsets, *, threshold: float = 0.5, quantile=None, p_out=None, b_out=None,
                tau_out=None, status=None, ws=None):
    """bllm_route with q = h Wq and k = h Wk formed inside the kernel (bf16 h, Wq, Wk)."""
    _dev(h, Wq, Wk, offsets)
    total, d = h.shape
    dev = h.device
    p_out = torch.empty(total, dtype=torch.float32, device=dev) if p_out is None else p_out
    b_out = torch.empty(total, dtype=torch.uint8, device=dev) if b_out is None else b_out
    tau_out = torch.empty(1, dtype=torch.float32, device=dev) if tau_out is None else tau_out
    w = _ws(route_workspace(total), ws, dev) if quantile is not None else ws
    rc = L.lib().bllm_route_fused(h.data_ptr(), Wq.data_ptr(), Wk.data_ptr(), _dt(h), d, offsets.data_ptr(),
                                  offsets.numel() - 1, total, float(threshold),
                                  -1.0 if quantile is None else float(quantile), p_out.data_ptr(),
                                  b_out.data_ptr(), tau_out.data_ptr(), _ptr(status), _ptr(w),
                                  0 if w is None else _nbytes(w), _stream())
    L.check("bllm_route_fused", rc)
    return p_out, b_out, tau_out


def compact(mask, offsets, *, rows=None, p=None, capacity=None, idx_out=None,
            chunk_offsets_out=None, rows_out=None, P_out=None, status=None, ws=None):
    """Keep set mask positions: returns (idx, chunk_offsets, rows_out, P_out, status).
    Outputs have `capacity` rows; the true count is chunk_offsets[-1] (on device)."""
    _dev(mask, offsets, rows, p)
    total = mask.numel()
    nseq = offsets.numel() - 1
    dev = mask.device
    cap = total if capacity is None else int(capacity)
    idx_out = torch.empty(max(cap, 1), dtype=torch.int32, device=dev) if idx_out is None else idx_out
    chunk_offsets_out = (torch.empty(nseq + 1, dtype=torch.int64, device=dev)
                         if chunk_offsets_out is None else chunk_offsets_out)
    d = 0
    dt = L.F32
    if rows is not None:
        d = rows.shape[1]
        dt = _dt(rows)
        if rows_out is None:
            rows_out = torch.empty((max(cap, 1), d), dtype=rows.dtype, device=dev)
    if p is not None and P_out is None:
        P_out = torch.empty(max(cap, 1), dtype=torch.float32, device=dev)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    w = _ws(compact_workspace(total), ws, dev)
    rc = L.lib().bllm_compact(mask.data_ptr(), _ptr(p), _ptr(rows), dt, d, offsets.data_ptr(), nseq,
                              total, cap, idx_out.data_ptr(), chunk_offsets_out.data_ptr(),
                              _ptr(rows_out), _ptr(P_out), status.data_ptr(), w.data_ptr(),
                              _nbytes(w), _stream())
    L.check("bllm_compact", rc)
    return idx_out, chunk_offsets_out, rows_out, P_out, status


def compact_noalloc(mask, offsets, *, rows=None, p=None, capacity=None, idx_out=None,
                    chunk_offsets_out=None, rows_out=None, P_out=None, status=None):
    """bllm_compact on the library's own scratch array (no workspace; at most
    2^27 positions).  Outputs must be passed in by a caller that cannot
    allocate; any left as None are allocated here for convenience."""
    _dev(mask, offsets, rows, p)
    total = mask.numel()
    nseq = offsets.numel() - 1
    dev = mask.device
    cap = total if capacity is None else int(capacity)
    idx_out = torch.empty(max(cap, 1), dtype=torch.int32, device=dev) if idx_out is None else idx_out
    chunk_offsets_out = (torch.empty(nseq + 1, dtype=torch.int64, device=dev)
                         if chunk_offsets_out is None else chunk_offsets_out)
    d = 0
    dt = L.F32
    if rows is not None:
        d = rows.shape[1]
        dt = _dt(rows)
        if rows_out is None:
            rows_out = torch.empty((max(cap, 1), d), dtype=rows.dtype, device=dev)
    if p is not None and P_out is None:
        P_out = torch.empty(max(cap, 1), dtype=torch.float32, device=dev)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    rc = L.lib().bllm_compact_noalloc(mask.data_ptr(), _ptr(p), _ptr(rows), dt, d, offsets.data_ptr(), nseq,
                                      total, cap, idx_out.data_ptr(), chunk_offsets_out.data_ptr(),
                                      _ptr(rows_out), _ptr(P_out), status.data_ptr(), _stream())
    L.check("bllm_compact_noalloc", rc)
    return idx_out, chunk_offsets_out, rows_out, P_out, status


def dechunk_ema(z, P, idx, chunk_offsets, offsets, total: int, *, out=None, ws=None,
                max_chunks=None):
    """EMA over chunks expanded back to `total` byte rows."""
    _dev(z, P, idx, chunk_offsets, offsets)
    d = z.shape[1]
    dev = z.device
    out = torch.empty((total, d), dtype=z.dtype, device=dev) if out is None else out
    w = _ws(dechunk_workspace(d), ws, dev)
    mc = z.shape[0] if max_chunks is None else int(max_chunks)
    rc = L.lib().bllm_dechunk_ema(z.data_ptr(), P.data_ptr(), _dt(z), d, idx.data_ptr(),
                                  chunk_offsets.data_ptr(), offsets.data_ptr(), offsets.numel() - 1,
                                  int(total), mc, out.data_ptr(), w.data_ptr(), _nbytes(w),
                                  _stream())
    L.check("bllm_dechunk_ema", rc)
    return out


def dechunk_ema_backward_workspace(d: int, max_chunks: int) -> int:
    return int(L.lib().bllm_dechunk_ema_backward_workspace(d, max_chunks))


def dechunk_ema_backward(z, P, dout, idx, chunk_offsets, offsets, *, dz_out=None, dP_out=None, ws=None,
                         max_chunks=None):
    """Gradients (dz, dP) of sum(dout * dechunk_ema(z, P, ...)) with respect to z and P."""
    _dev(z, P, dout, idx, chunk_offsets, offsets)
    d = z.shape[1]
    dev = z.device
    mc = z.shape[0] if max_chunks is None else int(max_chunks)
    dz_out = torch.empty((mc, d), dtype=z.dtype, device=dev) if dz_out is None else dz_out
    dP_out = torch.empty(mc, dtype=torch.float32, device=dev) if dP_out is None else dP_out
    w = _ws(dechunk_ema_backward_workspace(d, mc), ws, dev)
    rc = L.lib().bllm_dechunk_ema_backward(z.data_ptr(), P.data_ptr(), dout.data_ptr(), _dt(z), d,
                                           idx.data_ptr(), chunk_offsets.data_ptr(), offsets.data_ptr(),
                                           offsets.numel() - 1, dout.shape[0], mc, dz_out.data_ptr(),
                                           dP_out.data_ptr(), w.data_ptr(), _nbytes(w), _stream())
    L.check("bllm_dechunk_ema_backward", rc)
    return dz_out, dP_out


def coding_rate(h, eps2: float, *, dR_out=None, status=None, ws=None):
    """Delta R_t for h [nseq, T, d]; returns (dR fp32 [nseq, T], status)."""
    _dev(h)
    nseq, T, d = h.shape
    dev = h.device
    dR_out = torch.empty((nseq, T), dtype=torch.float32, device=dev) if dR_out is None else dR_out
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    w = _ws(coding_rate_workspace(nseq, T, d), ws, dev)
    rc = L.lib().bllm_coding_rate(h.data_ptr(), _dt(h), nseq, T, d, float(eps2), dR_out.data_ptr(),
                                  status.data_ptr(), w.data_ptr(), _nbytes(w), _stream())
    L.check("bllm_coding_rate", rc)
    return dR_out, status


def coding_rate_split(h, eps2: float, stream2, fork_event, join_event, *, dR_out=None, status=None, ws=None):
    """coding_rate with the batch's second half on `stream2` (a torch.cuda.Stream),
    forked and joined with the caller's two torch.cuda.Event objects."""
    _dev(h)
    nseq, T, d = h.shape
    dev = h.device
    dR_out = torch.empty((nseq, T), dtype=torch.float32, device=dev) if dR_out is None else dR_out
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    w = _ws(coding_rate_workspace(nseq, T, d), ws, dev)
    for ev in (fork_event, join_event):
        if not ev.cuda_event:  # torch creates the event at its first record
            ev.record()
    rc = L.lib().bllm_coding_rate_split(h.data_ptr(), _dt(h), nseq, T, d, float(eps2), dR_out.data_ptr(),
                                        status.data_ptr(), w.data_ptr(), _nbytes(w), _stream(),
                                        stream2.cuda_stream, fork_event.cuda_event, join_event.cuda_event)
    L.check("bllm_coding_rate_split", rc)
    return dR_out, status


def coding_rate_stream(h, eps2: float, state_in=None, *, state_out=None, want_state=True, dR_out=None,
                       status=None, ws=None):
    """Delta R_t of one window h [nseq, W, d] of a stream, given the carried
    prefix matrix state_in (fp32 [nseq, d, d]; None at the stream's start).
    Returns (dR fp32 [nseq, W], state_out fp32 [nseq, d, d] or None, status);
    state_out may be state_in itself (updated in place); want_state=False
    skips the next carry."""
    _dev(h)
    nseq, W, d = h.shape
    dev = h.device
    dR_out = torch.empty((nseq, W), dtype=torch.float32, device=dev) if dR_out is None else dR_out
    if not want_state:
        state_out = None
    elif state_out is None:
        state_out = torch.empty((nseq, d, d), dtype=torch.float32, device=dev)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    w = _ws(coding_rate_workspace(nseq, W, d), ws, dev)
    rc = L.lib().bllm_coding_rate_stream(h.data_ptr(), _dt(h), nseq, W, d, float(eps2), _ptr(state_in),
                                         _ptr(state_out), dR_out.data_ptr(), status.data_ptr(),
                                         w.data_ptr(), _nbytes(w), _stream())
    L.check("bllm_coding_rate_stream", rc)
    return dR_out, state_out, status


def topk_select(score, K: int, *, idx_out=None, mask_out=None, status=None, want_mask=True):
    """BOS + Top-(K-1) positions per sequence in time order: (idx int32, mask uint8, status)."""
    _dev(score)
    nseq, T = score.shape
    dev = score.device
    idx_out = torch.empty((nseq, K), dtype=torch.int32, device=dev) if idx_out is None else idx_out
    if want_mask and mask_out is None:
        mask_out = torch.empty((nseq, T), dtype=torch.uint8, device=dev)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    rc = L.lib().bllm_topk_select(score.data_ptr(), nseq, T, int(K), idx_out.data_ptr(),
                                  _ptr(mask_out), status.data_ptr(), _stream())
    L.check("bllm_topk_select", rc)
    return idx_out, mask_out, status


def gather_topk(h, idx, *, z_out=None):
    """z [nseq, K, d] = the rows of h [nseq, T, d] at the positions idx [nseq, K] (int32)."""
    _dev(h, idx)
    nseq, T, d = h.shape
    K = idx.shape[1]
    if idx.dtype != torch.int32 or idx.shape[0] != nseq:
        raise ValueError("idx must be int32 [nseq, K]")
    z_out = torch.empty((nseq, K, d), dtype=h.dtype, device=h.device) if z_out is None else z_out
    rc = L.lib().bllm_gather_topk(h.data_ptr(), _dt(h), nseq, T, d, K, idx.data_ptr(), z_out.data_ptr(),
                                  _stream())
    L.check("bllm_gather_topk", rc)
    return z_out


def topk_select_window(score, K: int, first: bool, *, idx_out=None, mask_out=None, status=None, want_mask=True):
    """Local Top-K of one window [nseq, W] of a stream: the first window as
    ``topk_select`` (BOS + K-1), later windows their K largest scores."""
    _dev(score)
    nseq, W = score.shape
    dev = score.device
    idx_out = torch.empty((nseq, K), dtype=torch.int32, device=dev) if idx_out is None else idx_out
    if want_mask and mask_out is None:
        mask_out = torch.empty((nseq, W), dtype=torch.uint8, device=dev)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    rc = L.lib().bllm_topk_select_window(score.data_ptr(), nseq, W, int(K), 1 if first else 0, idx_out.data_ptr(),
                                         _ptr(mask_out), status.data_ptr(), _stream())
    L.check("bllm_topk_select_window", rc)
    return idx_out, mask_out, status


def upsample_plan(idx, T: int, nbins: int, *, ws=None, d_global: int = 8, d_local: int = 8):
    """The upsample's work items from the chunk starts idx int32 [nseq, K] into a
    workspace (returned; pass it to ``upsample_apply``)."""
    _dev(idx)
    nseq, K = idx.shape
    w = _ws(upsample_workspace(nseq, T, K, d_global, d_local, nbins), ws, idx.device)
    rc = L.lib().bllm_upsample_plan(idx.data_ptr(), nseq, int(T), K, int(nbins), w.data_ptr(), _nbytes(w),
                                    _stream())
    L.check("bllm_upsample_plan", rc)
    return w


def upsample_apply(g, W, h, nbins: int, ws, *, s_out=None):
    """s_t = h_t + g_{c(t)} W_{bin(t)} from a plan made by ``upsample_plan`` in ws."""
    _dev(g, W, h, ws)
    nseq, K, dg = g.shape
    T, dl = h.shape[1], h.shape[2]
    s_out = torch.empty_like(h) if s_out is None else s_out
    rc = L.lib().bllm_upsample_apply(g.data_ptr(), W.data_ptr(), h.data_ptr(), _dt(h), nseq, T, K, dg, dl,
                                     int(nbins), s_out.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream())
    L.check("bllm_upsample_apply", rc)
    return s_out


def upsample_bins(g, W, idx, h, nbins: int, *, s_out=None, ws=None):
    """s_t = h_t + g_{c(t)} W_{bin(t)}; g [nseq,K,dg], W [nbins,dg,dl], idx int32 [nseq,K], h [nseq,T,dl]."""
    _dev(g, W, idx, h)
    nseq, K, dg = g.shape
    T, dl = h.shape[1], h.shape[2]
    dev = h.device
    s_out = torch.empty_like(h) if s_out is None else s_out
    w = _ws(upsample_workspace(nseq, T, K, dg, dl, nbins), ws, dev)
    rc = L.lib().bllm_upsample_bins(g.data_ptr(), W.data_ptr(), idx.data_ptr(), h.data_ptr(), _dt(h),
                                    nseq, T, K, dg, dl, int(nbins), s_out.data_ptr(), w.data_ptr(),
                                    _nbytes(w), _stream())
    L.check("bllm_upsample_bins", rc)
    return s_out
