"""ctypes loader for libbllm.so (the C ABI declared in include/bllm.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any operation.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("BLLM_LIB", os.path.join(_HERE, "libbllm.so"))

OK, E_INVAL, E_NOTSUP, E_WS, E_HIP = 0, -1, -2, -3, -4
S_CAPACITY, S_NONFINITE, S_INCOMPLETE = 1, 2, 4
F32, BF16 = 0, 1

_p = C.c_void_p
_i64 = C.c_int64
_SIGS = {
    "bllm_version": (C.c_int, []),
    "bllm_status_string": (C.c_char_p, [C.c_int]),
    "bllm_route_workspace": (C.c_size_t, [_i64]),
    "bllm_route": (C.c_int, [_p, _p, C.c_int, _i64, _p, _i64, _i64, C.c_float, C.c_double,
                             _p, _p, _p, _p, _p, C.c_size_t, _p]),
    "bllm_route_fused": (C.c_int, [_p, _p, _p, C.c_int, _i64, _p, _i64, _i64, C.c_float, C.c_double,
                                   _p, _p, _p, _p, _p, C.c_size_t, _p]),
    "bllm_compact_workspace": (C.c_size_t, [_i64]),
    "bllm_compact": (C.c_int, [_p, _p, _p, C.c_int, _i64, _p, _i64, _i64, _i64, _p, _p, _p, _p,
                               _p, _p, C.c_size_t, _p]),
    "bllm_compact_noalloc": (C.c_int, [_p, _p, _p, C.c_int, _i64, _p, _i64, _i64, _i64, _p, _p, _p, _p,
                                       _p, _p]),
    "bllm_dechunk_workspace": (C.c_size_t, [_i64]),
    "bllm_dechunk_ema": (C.c_int, [_p, _p, C.c_int, _i64, _p, _p, _p, _i64, _i64, _i64, _p, _p,
                                   C.c_size_t, _p]),
    "bllm_dechunk_ema_backward_workspace": (C.c_size_t, [_i64, _i64]),
    "bllm_dechunk_ema_backward": (C.c_int, [_p, _p, _p, C.c_int, _i64, _p, _p, _p, _i64, _i64, _i64,
                                            _p, _p, _p, C.c_size_t, _p]),
    "bllm_coding_rate_workspace": (C.c_size_t, [_i64, _i64, _i64]),
    "bllm_coding_rate": (C.c_int, [_p, C.c_int, _i64, _i64, _i64, C.c_double, _p, _p, _p,
                                   C.c_size_t, _p]),
    "bllm_coding_rate_split": (C.c_int, [_p, C.c_int, _i64, _i64, _i64, C.c_double, _p, _p, _p, C.c_size_t, _p,
                                         _p, _p, _p]),
    "bllm_coding_rate_stream": (C.c_int, [_p, C.c_int, _i64, _i64, _i64, C.c_double, _p, _p, _p, _p, _p,
                                          C.c_size_t, _p]),
    "bllm_topk_select": (C.c_int, [_p, _i64, _i64, _i64, _p, _p, _p, _p]),
    "bllm_topk_select_window": (C.c_int, [_p, _i64, _i64, _i64, C.c_int, _p, _p, _p, _p]),
    "bllm_gather_topk": (C.c_int, [_p, C.c_int, _i64, _i64, _i64, _i64, _p, _p, _p]),
    "bllm_upsample_workspace": (C.c_size_t, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "bllm_upsample_plan": (C.c_int, [_p, _i64, _i64, _i64, _i64, _p, C.c_size_t, _p]),
    "bllm_upsample_apply": (C.c_int, [_p, _p, _p, C.c_int, _i64, _i64, _i64, _i64, _i64, _i64, _p, _p,
                                      C.c_size_t, _p]),
    "bllm_upsample_bins": (C.c_int, [_p, _p, _p, _p, C.c_int, _i64, _i64, _i64, _i64, _i64, _i64,
                                     _p, _p, C.c_size_t, _p]),
}
EXPORTS = tuple(_SIGS)

_lib = None


class BllmError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({status_string(code)})")
        self.code = code


def lib() -> C.CDLL:
    """Load libbllm.so once; raise if it is missing (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not built: run `python -m byte_level_lm_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().bllm_status_string(int(code)).decode()


def check(fn: str, code: int) -> None:
    if code != OK:
        raise BllmError(fn, code)
