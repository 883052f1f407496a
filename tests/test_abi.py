"""The C-ABI library loads and exports every symbol include/bllm.h declares;
host-side argument checks return errors before anything is enqueued."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bllm.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(bllm_\w+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    from byte_level_lm_amd import _lib
    return _lib.lib()


def test_every_declared_symbol_is_exported_and_bound(L):
    from byte_level_lm_amd import _lib
    decl = _declared()
    assert len(decl) >= 13
    for name in decl:
        assert hasattr(L, name), name
    assert sorted(_lib.EXPORTS) == decl


def test_version_and_status_strings(L):
    assert L.bllm_version() >= 100
    assert L.bllm_status_string(0) == b"ok"
    assert b"invalid" in L.bllm_status_string(-1)
    assert L.bllm_status_string(-3).startswith(b"workspace")


def test_workspace_sizes(L):
    assert L.bllm_route_workspace(1000) > 2048 * 4
    assert L.bllm_compact_workspace(10**6) >= (10**6 // 4096) * 4
    # per tile: one fp32 product plus d fp32 aggregate and d fp32 carry values
    w512, w768 = L.bllm_dechunk_workspace(512), L.bllm_dechunk_workspace(768)
    tiles = (w768 - w512) // (2 * 256 * 4)
    assert tiles >= 256 and w512 >= tiles * (1 + 2 * 512) * 4
    # d = 512: blocks of c = 256 rows, 32 blocks per sequence, block matrices of
    # (512 + 256)^2 fp32 plus a 64 x 64 inverse slot each
    assert L.bllm_coding_rate_workspace(32, 8192, 512) == 32 * 32 * (768 * 768 + 2 * 64 * 64) * 4 + 256
    assert L.bllm_coding_rate_workspace(0, 8192, 512) == 0
    # at most T + T/32 + 1 work items per sequence (one per present bin, one
    # more per 32 positions of a run), 16 bytes each
    assert L.bllm_upsample_workspace(32, 8192, 2048, 1536, 512, 16) >= 32 * (8192 + 256 + 1) * 16


def test_argument_errors_return_before_any_launch(L):
    dummy = C.c_void_p(16)
    # null q
    assert L.bllm_route(None, dummy, 0, 64, dummy, 1, 10, 0.5, -1.0, dummy, dummy, None, None, None, 0, None) == -1
    # bad dtype
    assert L.bllm_route(dummy, dummy, 7, 64, dummy, 1, 10, 0.5, -1.0, dummy, dummy, None, None, None, 0, None) == -2
    # d*e not a multiple of 16 bytes
    assert L.bllm_route(dummy, dummy, 0, 3, dummy, 1, 10, 0.5, -1.0, dummy, dummy, None, None, None, 0, None) == -2
    # quantile mode without workspace
    assert L.bllm_route(dummy, dummy, 0, 64, dummy, 1, 10, 0.5, 0.75, dummy, dummy, None, None, None, 0, None) == -3
    # compact: negative capacity, missing rows_out
    assert L.bllm_compact(dummy, None, None, 0, 0, dummy, 1, 10, -1, dummy, dummy, None, None, None, dummy, 1 << 20, None) == -1
    assert L.bllm_compact(dummy, None, dummy, 0, 64, dummy, 1, 10, 5, dummy, dummy, None, None, None, dummy, 1 << 20, None) == -1
    # coding rate: eps2 <= 0, d too large, workspace too small
    assert L.bllm_coding_rate(dummy, 0, 1, 8, 8, 0.0, dummy, None, dummy, 1 << 30, None) == -1
    assert L.bllm_coding_rate(dummy, 0, 1, 8, 1024, 0.5, dummy, None, dummy, 1 << 30, None) == -2
    assert L.bllm_coding_rate(dummy, 0, 1, 64, 8, 0.5, dummy, None, dummy, 16, None) == -3
    # split coding rate: no second stream or events, second stream equal to the first
    assert L.bllm_coding_rate_split(dummy, 0, 2, 64, 8, 0.5, dummy, None, dummy, 1 << 30, None, None, dummy,
                                    dummy) == -1
    assert L.bllm_coding_rate_split(dummy, 0, 2, 64, 8, 0.5, dummy, None, dummy, 1 << 30, dummy, dummy, dummy,
                                    dummy) == -1
    assert L.bllm_coding_rate_split(dummy, 0, 2, 64, 8, 0.5, dummy, None, dummy, 1 << 30, None, dummy, None,
                                    dummy) == -1
    # top-k: K > T, K < 1, T above 65536
    assert L.bllm_topk_select(dummy, 1, 10, 11, dummy, None, None, None) == -1
    assert L.bllm_topk_select(dummy, 1, 10, 0, dummy, None, None, None) == -1
    assert L.bllm_topk_select(dummy, 1, 70000, 5, dummy, None, None, None) == -2
    assert L.bllm_coding_rate_stream(dummy, 0, 1, 8, 8, 0.0, None, None, dummy, None, dummy, 1 << 30, None) == -1
    assert L.bllm_coding_rate_stream(None, 0, 1, 8, 8, 0.5, dummy, dummy, dummy, None, dummy, 1 << 30, None) == -1
    assert L.bllm_coding_rate_stream(dummy, 0, 1, 8, 1024, 0.5, None, dummy, dummy, None, dummy, 1 << 30, None) == -2
    assert L.bllm_coding_rate_stream(dummy, 0, 1, 64, 8, 0.5, dummy, dummy, dummy, None, dummy, 16, None) == -3
    assert L.bllm_topk_select_window(dummy, 1, 10, 11, 0, dummy, None, None, None) == -1
    assert L.bllm_topk_select_window(dummy, 1, 10, 0, 1, dummy, None, None, None) == -1
    assert L.bllm_topk_select_window(dummy, 1, 70000, 5, 0, dummy, None, None, None) == -2
    # upsample: fp32 unsupported, nbins < 1
    assert L.bllm_upsample_bins(dummy, dummy, dummy, dummy, 0, 1, 64, 4, 64, 32, 16, dummy, dummy, 1 << 30, None) == -2
    assert L.bllm_upsample_bins(dummy, dummy, dummy, dummy, 1, 1, 64, 4, 64, 32, 0, dummy, dummy, 1 << 30, None) == -1
    # upsample plan / apply: K > T, null idx, fp32 unsupported, workspace too small
    assert L.bllm_upsample_plan(dummy, 1, 64, 65, 16, dummy, 1 << 30, None) == -1
    assert L.bllm_upsample_plan(None, 1, 64, 4, 16, dummy, 1 << 30, None) == -1
    assert L.bllm_upsample_plan(dummy, 1, 64, 4, 16, dummy, 16, None) == -3
    assert L.bllm_upsample_apply(dummy, dummy, dummy, 0, 1, 64, 4, 64, 32, 16, dummy, dummy, 1 << 30, None) == -2
    assert L.bllm_upsample_apply(dummy, dummy, None, 1, 1, 64, 4, 64, 32, 16, dummy, dummy, 1 << 30, None) == -1
    assert L.bllm_upsample_apply(dummy, dummy, dummy, 1, 1, 64, 4, 64, 32, 16, dummy, dummy, 16, None) == -3
    # an invalid argument is reported before an unsupported one (K > T with an fp32 dtype)
    assert L.bllm_upsample_bins(dummy, dummy, dummy, dummy, 0, 1, 64, 65, 64, 32, 16, dummy, dummy, 1 << 30,
                                None) == -1
    # Top-K gather: K > T, null idx, rows not a multiple of 16 bytes
    assert L.bllm_gather_topk(dummy, 0, 1, 10, 8, 11, dummy, dummy, None) == -1
    assert L.bllm_gather_topk(dummy, 0, 1, 10, 8, 4, None, dummy, None) == -1
    assert L.bllm_gather_topk(dummy, 1, 1, 10, 4, 4, dummy, dummy, None) == -2
    # compact without a workspace: more positions than its scratch holds (checked before any HIP call)
    assert L.bllm_compact_noalloc(dummy, None, None, 0, 0, dummy, 1, (1 << 27) + 1, 5, dummy, dummy, None, None,
                                  None, None) == -3
    assert L.bllm_compact_noalloc(dummy, None, None, 0, 0, dummy, 1, 10, -1, dummy, dummy, None, None,
                                  None, None) == -1
    # dechunk: null P
    assert L.bllm_dechunk_ema(dummy, None, 1, 512, dummy, dummy, dummy, 1, 10, 10, dummy, dummy, 1 << 30, None) == -1
    # fused route: fp32 unsupported, d not a multiple of 128
    assert L.bllm_route_fused(dummy, dummy, dummy, 0, 512, dummy, 1, 10, 0.5, -1.0, dummy, dummy, None, None, None, 0, None) == -2
    assert L.bllm_route_fused(dummy, dummy, dummy, 1, 192, dummy, 1, 10, 0.5, -1.0, dummy, dummy, None, None, None, 0, None) == -2
    # dechunk backward: null dout, workspace too small
    assert L.bllm_dechunk_ema_backward(dummy, dummy, None, 1, 512, dummy, dummy, dummy, 1, 10, 10, dummy, dummy,
                                       dummy, 1 << 30, None) == -1
    assert L.bllm_dechunk_ema_backward(dummy, dummy, dummy, 1, 512, dummy, dummy, dummy, 1, 10, 10, dummy, dummy,
                                       dummy, 16, None) == -3


def test_product_path_does_not_touch_the_oracle():
    """No module of the package imports, names or reads oracle/."""
    pkg = os.path.join(ROOT, "byte_level_lm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", txt), os.path.join(dirpath, f)
