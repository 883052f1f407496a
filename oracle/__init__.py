"""CPU oracle for the dynamic-chunking layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 numpy implementations of what the chunk layer computes,
written from the pages' statement of the method.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package; the product path
(``byte_level_lm_amd``) never does, and this package imports nothing from it.

Sources (page titles; sections named as on the page):
  [BG]  "ByteGen: A Tokenizer-Free Generative Model for Orderbook Events in
        Byte Space" analyst report, section 2.3 Methodology (H-Net dynamic
        chunking: cosine similarity of adjacent byte representations gives a
        boundary probability, EMA smoothing makes the boundaries
        differentiable; two stages compress to 1/4 and 1/16).
  [BF2] "ByteFlow: Language Modeling through Adaptive Byte Compression
        without a Tokenizer" paper notes (ICLR 2026), key designs 2 (coding
        rate chunking, Top-K with BOS) and 4 (upsampling by relative position
        in the chunk with shared bin matrices, large residual).
  [BF4] the ByteFlow paper page (arXiv 2603.03583): "prerequisites / lossy
        coding rate" (R_eps formula), "method step details" stages 2 and 4
        (Delta R, S = {1} + Top-(K-1) in time order, chunk map c(t), bins,
        residual), "independent analysis of weaknesses" (incremental
        Sherman-Morrison-Woodbury evaluation suggested; streaming inference
        by a sliding window with a local Top-K suggested).

Where the pages are silent the reading taken is stated in the docstring of
the function concerned.  [BG] describes H-Net routing and the EMA only in
words; the formulas used are the plainest ones that description supports:
p_t = (1 - cos(q_t, k_{t-1}))/2 with p = 1 at a sequence start, b_t = p_t >= tau,
and zbar_t = P_t z_t + (1 - P_t) zbar_{t-1}.

Every function here is pinned by tests against something other than itself
(closed forms, brute force on tiny inputs, library routines, invariants);
none is "parity unpinned".
"""
from .hnet import route, boundary_mask, stage_quantile, compact, dechunk_ema, dechunk_ema_backward  # noqa: F401
from .byteflow import (  # noqa: F401
    alpha_of, coding_rate, coding_rate_at, coding_rate_stream, topk_select, topk_select_window, topk_mask, gather, chunk_bins, upsample_bins,
)
