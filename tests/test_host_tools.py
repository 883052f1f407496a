"""Host-side logic of bench.py and of the rocprofv3 summary tool (no GPU)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from byte_level_lm_amd import profsum  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_op_rates_fractions():
    d = bench.op_rates({"bytes": 8e9, "flops": 157.3e12 * 1e-3, "peak_tflops": bench.FP32_MFMA_PEAK_TFLOPS}, 2.0)
    assert d["ms"] == 2.0
    assert d["hbm_GBps"] == pytest.approx(4000.0) and d["hbm_frac"] == pytest.approx(0.5)
    assert d["TFLOPs"] == pytest.approx(78.65) and d["mfma_frac"] == pytest.approx(0.5)
    # contractions without a stated type are priced at the bf16 peak
    d = bench.op_rates({"flops": 2.5e9}, 1.0)
    assert d["mfma_peak"] == bench.BF16_MFMA_PEAK_TFLOPS and d["mfma_frac"] == pytest.approx(1e-3)


def test_step_roofline_sums_op_ideals():
    alg = {"hbm op": {"bytes": 8e9},  # 1 ms at 8 TB/s
           "coding_rate": {"flops": 3e12, "bytes": 1.0},  # 2e12 at bf16 peak + 1e12 at fp32 peak
           "upsample_bins": {"flops": 2.5e12, "bytes": 4e9}}  # 1 ms of MFMA beats 0.5 ms of HBM
    want = 1.0 + (2e12 / 2.5e15 + 1e12 / 157.3e12) * 1e3 + 1.0
    r = bench.step_roofline(alg, 20.0)
    assert r["ideal_ms"] == pytest.approx(want, rel=1e-3) and r["frac"] == pytest.approx(want / 20.0, rel=1e-3)


def test_coding_rate_traffic_tracks_the_sources():
    """The committed counter summary is used only while it matches the kernel sources."""
    path = os.path.join(ROOT, "profiles", "coding_rate_bf16_32x8192x512.md")
    text = open(path).read()
    block = json.loads(text.split("```json\n")[-1].split("\n```")[0])
    t = bench.coding_rate_traffic()
    if block["sources_sha256"] == profsum.sources_sha256("coding_rate"):
        assert t == block["hbm_bytes_per_call"] and t > 0
    else:
        assert t is None


def _write_trace(path, kernels):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, s, e in kernels:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": s, "End_Timestamp": e})


def test_profsum_groups_calls_and_keeps_the_last(tmp_path):
    gram = "bllm::(anonymous namespace)::cr_gram_prefix_bf16(unsigned short const*)"
    diag = "bllm::(anonymous namespace)::cr_diag(float*)"
    panel = "void bllm::(anonymous namespace)::cr_panel<1>(void const*)"
    other = "at::native::elementwise_kernel"
    ks = []
    t = 0
    # a set-up call of 1000 ns per kernel, then two profiled calls of 100 and 300 ns per kernel
    for per in (1000, 100, 300):
        for name in (gram, diag, panel, other, panel):
            ks.append((name, t, t + per))
            t += per + 10
    d = tmp_path / "trace"
    d.mkdir()
    _write_trace(d / "x_kernel_trace.csv", ks)
    calls = profsum.trace_calls("coding_rate", str(d))
    assert [len(c) for c in calls] == [4, 4, 4]  # the unrelated kernel is not part of a call
    out = tmp_path / "sum.md"
    sys_argv = sys.argv
    try:
        sys.argv = ["profsum", "--op", "coding_rate", "--last", "2", "--trace", str(d), "--cmd", "c",
                    "--workload", "w", "--out", str(out)]
        profsum.main()
    finally:
        sys.argv = sys_argv
    text = out.read_text()
    assert "Calls profiled: 2" in text
    block = json.loads(text.split("```json\n")[-1].split("\n```")[0])
    assert block["kernel_us_per_call"] == pytest.approx(4 * 200 / 1e3)
    assert block["sources_sha256"] == profsum.sources_sha256("coding_rate")


def test_profsum_calls_split_over_two_streams(tmp_path):
    """A call made of two halves on two streams: its kernels interleave in
    time, both halves' first kernels open the same call, the span runs from
    the first start to the last end, and the counters of the last call start
    at its first half's first dispatch."""
    gram = "bllm::(anonymous namespace)::cr_gram_prefix_bf16(unsigned short const*)"
    diag = "bllm::(anonymous namespace)::cr_diag(float*)"
    panel = "void bllm::(anonymous namespace)::cr_panel<1>(void const*)"
    ks, t = [], 0
    ks.append((gram, 0, 50))  # a set-up call on one stream
    ks.append((diag, 60, 70))
    t = 1000
    for _ in range(2):  # two calls, each: half A and half B overlapping
        ks += [(gram, t, t + 100), (gram, t + 5, t + 110), (diag, t + 100, t + 120), (diag, t + 110, t + 125),
               (panel, t + 120, t + 300), (panel, t + 125, t + 320)]
        t += 1000
    d = tmp_path / "trace"
    d.mkdir()
    _write_trace(d / "x_kernel_trace.csv", ks)
    calls = profsum.trace_calls("coding_rate", str(d), parts=2)
    assert [len(c) for c in calls] == [2, 6, 6]
    out = tmp_path / "sum.md"
    # counters: dispatch ids in order of enqueue (half A's kernels, then half B's)
    cdir = tmp_path / "pmc"
    cdir.mkdir()
    names = [gram, diag] + [gram, diag, panel, gram, diag, panel] * 2
    with open(cdir / "x_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, n in enumerate(names):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": n, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1 + i})
    assert profsum.counter_last_call("coding_rate", str(cdir), "FETCH_SIZE", parts=2) == sum(range(9, 15))
    sys_argv = sys.argv
    try:
        sys.argv = ["profsum", "--op", "coding_rate", "--parts", "2", "--last", "2", "--trace", str(d), "--cmd", "c",
                    "--workload", "w", "--out", str(out)]
        profsum.main()
    finally:
        sys.argv = sys_argv
    block = json.loads(out.read_text().split("```json\n")[-1].split("\n```")[0])
    assert block["us_per_call"] == pytest.approx(0.32) and block["parts"] == 2
    assert block["kernel_us_per_call"] == pytest.approx((100 + 105 + 20 + 15 + 180 + 195) / 1e3, abs=0.01)


def test_profsum_step_timeline_keeps_kernels_still_running(tmp_path):
    """The timeline of the last step starts at its first Gram-prefix kernel
    and keeps a kernel of the step before that still runs at that time
    (negative start), but not one that ended before it."""
    gram = "bllm::(anonymous namespace)::cr_gram_prefix_bf16(unsigned short const*)"
    expand = "void bllm::(anonymous namespace)::ema_tile_expand<1>(void const*)"
    topk = "void bllm::(anonymous namespace)::topk_kernel<true>(float const*)"
    ks = [(gram, 0, 100), (gram, 5, 110), (expand, 900, 950), (expand, 960, 1030),
          (gram, 1000, 1100), (gram, 1005, 1120), (topk, 1200, 1230)]
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "x_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Queue_Id"])
        w.writeheader()
        for name, s0, s1 in ks:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": s0, "End_Timestamp": s1, "Queue_Id": 1})
    out = tmp_path / "tl.md"
    sys_argv = sys.argv
    try:
        sys.argv = ["profsum", "--op", "step-timeline", "--trace", str(d), "--cmd", "c", "--workload", "w",
                    "--out", str(out)]
        profsum.main()
    finally:
        sys.argv = sys_argv
    rows = [ln for ln in out.read_text().splitlines() if ln.startswith("| ") and "kernel |" not in ln]
    assert len(rows) == 4  # the still-running expand, both Grams, Top-K
    assert rows[0].startswith("| -0.0") and "ema_tile_expand" in rows[0]
    assert "topk_kernel" in rows[-1]
