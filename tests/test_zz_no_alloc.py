"""bllm_compact_noalloc (no workspace argument: the library's own scratch
array) against bllm_compact with a workspace, bit for bit, on two calls in a
row, the second with a smaller input."""
import numpy as np
import pytest

from tests.helpers import say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _inputs(rng, lengths, d):
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = int(off[-1])
    mask = (rng.random(N) < 0.3).astype(np.uint8)
    mask[off[:-1][np.asarray(lengths) > 0]] = 1
    p = rng.random(N).astype(np.float32)
    rows = rng.standard_normal((N, d)).astype(np.float32)
    return off, mask, p, rows


def _run(fn, noalloc, off, mask, p, rows, cap):
    import torch
    import byte_level_lm_amd as B
    from byte_level_lm_amd import _lib
    N, d = rows.shape
    nseq = len(off) - 1
    md, od, pd = to_dev(mask), to_dev(off), to_dev(p)
    rd = to_dev(rows).to(torch.bfloat16)
    idx = torch.full((max(cap, 1),), -1, dtype=torch.int32, device="cuda")
    co = torch.full((nseq + 1,), -1, dtype=torch.int64, device="cuda")
    ro = torch.zeros((max(cap, 1), d), dtype=torch.bfloat16, device="cuda")
    Po = torch.full((max(cap, 1),), -1.0, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    args = [md.data_ptr(), pd.data_ptr(), rd.data_ptr(), _lib.BF16, d, od.data_ptr(), nseq, N, cap,
            idx.data_ptr(), co.data_ptr(), ro.data_ptr(), Po.data_ptr(), st.data_ptr()]
    if noalloc:
        rc = fn(*args, stream)
    else:
        ws = torch.empty(B.compact_workspace(N), dtype=torch.uint8, device="cuda")
        rc = fn(*args, ws.data_ptr(), ws.numel(), stream)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return [to_np(x) for x in (idx, co, ro, Po, st)]


def test_compact_noalloc_matches_compact_twice():
    import byte_level_lm_amd as B
    L = B.lib()
    f = L.bllm_compact_noalloc
    rng = np.random.default_rng(90)
    cases = [([70000, 0, 123457, 4096, 99999, 1], 512, None), ([3000, 17, 0, 2500], 64, 900)]
    for lengths, d, cap in cases:
        off, mask, p, rows = _inputs(rng, lengths, d)
        c = int(off[-1]) if cap is None else cap
        say("compact noalloc: positions", int(off[-1]), "d", d, "capacity", c)
        want = _run(L.bllm_compact, False, off, mask, p, rows, c)
        got = _run(f, True, off, mask, p, rows, c)
        for a, b_ in zip(want, got):
            assert np.array_equal(a, b_, equal_nan=True)
        M = int(want[1][-1])
        assert M == int(mask.sum())
        if cap is not None:
            assert M > cap and int(got[4][0]) & 1  # capacity flag in both
