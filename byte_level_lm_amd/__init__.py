"""MI355X-native dynamic-chunking layer for tokenizer-free hierarchical byte models.

The compute path is the HIP library libbllm.so (C ABI in include/bllm.h);
this package only marshals torch tensors (device memory and the current
stream) into it.  See ``byte_level_lm_amd.ops``.
"""
from ._lib import lib, LIB_PATH, EXPORTS, BllmError  # noqa: F401
from .ops import (  # noqa: F401
    route, route_fused, compact, compact_noalloc, dechunk_ema, dechunk_ema_backward, coding_rate, coding_rate_split, coding_rate_stream, topk_select,
    topk_select_window, gather_topk, upsample_bins, upsample_plan, upsample_apply,
    route_workspace, compact_workspace, dechunk_workspace, dechunk_ema_backward_workspace,
    coding_rate_workspace, upsample_workspace,
)
