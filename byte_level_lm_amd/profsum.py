"""Summaries of rocprofv3 runs of bench.py, written as short markdown files.

    python -m byte_level_lm_amd.profsum --op coding_rate --trace DIR \
        [--fetch DIR --write DIR --copy-fetch DIR --copy-write DIR] \
        --cmd "the rocprofv3 commands" --workload "..." --out profiles/NAME.md
    python -m byte_level_lm_amd.profsum --op step --trace DIR --cmd ... --workload ... --out ...

DIR is a rocprofv3 ``--output-format csv`` directory.  ``--trace`` holds a
``--kernel-trace --stats`` run; ``--fetch``/``--write`` hold ``--pmc FETCH_SIZE``
and ``--pmc WRITE_SIZE`` runs of the same op; ``--copy-*`` the same counters
for ``bench.py --profile-op copy`` (a device copy of ``bench.COPY_BYTES``),
which calibrates KiB-per-dispatch counter values into bytes.

The summary ends with a JSON block (op, per-call duration, HBM bytes per call,
SHA-256 of the op's sources) that bench.py reads for its roofline traffic; it
ignores the block once the sources have changed.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))

# kernels that make up one call of each C-ABI op, and the sources they come from
OPS = {
    "coding_rate": (("cr_gram_prefix", "cr_diag", "cr_panel"), ("coding_rate.hip", "common.h")),
    "upsample_bins": (("up_count", "up_offsets", "up_items", "up_transpose", "up_gemm"),
                      ("upsample.hip", "common.h")),
}


def sources_sha256(op: str) -> str:
    h = hashlib.sha256()
    for name in OPS[op][1]:
        with open(os.path.join(HERE, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _short(name: str) -> str:
    n = name.split("(anonymous namespace)::", 1)[1] if "(anonymous namespace)::" in name else name
    return n.split("(")[0].replace("void ", "").strip()


def _one(d: str, pattern: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return hits[0]


def _of_op(op: str, name: str) -> bool:
    return any(_short(name).startswith(p) for p in OPS[op][0])


def trace_calls(op: str, d: str, parts: int = 1):
    """Kernel dispatches of the op grouped into calls.  A call starts at its
    first kernel; a call that runs as `parts` halves on several streams has
    `parts` first kernels, which are grouped in runs of `parts` counted from the
    end of the run (the profiled calls are the last ones)."""
    rows = list(csv.DictReader(open(_one(d, "*kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    rows = [r for r in rows if _of_op(op, r["Kernel_Name"])]
    first = OPS[op][0][0]
    heads = [i for i, r in enumerate(rows) if _short(r["Kernel_Name"]).startswith(first)]
    keep = set(heads[len(heads) % parts::parts]) if parts > 1 else set(heads)
    calls = []
    for i, r in enumerate(rows):
        if i in keep or not calls:
            calls.append([])
        calls[-1].append(r)
    return calls


def counter_last_call(op: str, d: str, counter: str, parts: int = 1) -> float:
    """Sum of a counter (KiB) over the kernels of the op's last call in a --pmc
    run (dispatch ids follow the order of enqueue, so a call made of `parts`
    halves starts at the `parts`-th first kernel from the end)."""
    rows = list(csv.DictReader(open(_one(d, "*counter_collection.csv"))))
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = int(r["Dispatch_Id"])
        per.setdefault(key, [r["Kernel_Name"], 0.0])
        per[key][1] += float(r["Counter_Value"])
    disp = sorted(per.items())
    first = OPS[op][0][0]
    starts = [i for i, (_, (n, _)) in enumerate(disp) if _short(n).startswith(first)]
    if len(starts) < parts:
        raise ValueError(f"fewer than {parts} {first} dispatches in {d}")
    return sum(v for _, (n, v) in disp[starts[-parts]:] if _of_op(op, n))


def counter_copy(d: str, counter: str) -> float:
    rows = list(csv.DictReader(open(_one(d, "*counter_collection.csv"))))
    vals = {}
    for r in rows:
        if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]:
            vals[int(r["Dispatch_Id"])] = vals.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    if not vals:
        raise ValueError(f"no copy dispatch with {counter} in {d}")
    return vals[max(vals)]


def step_summary(d: str, cmd: str, workload: str, out: str, top: int = 25):
    """Per-kernel table of a whole run (kernel_stats.csv), longest total first."""
    rows = list(csv.DictReader(open(_one(d, "*kernel_stats.csv"))))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 summary: {workload}", "", "Command (run from the repository root on the GPU host):", "",
             "```", cmd, "```", "", "| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
    for r in rows[:top]:
        lines.append(f"| {_short(r['Name'])[:60]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# the kernels that open each op of a bench.py step, in step order (the H-Net
# stage and dechunk ops appear twice: stage 1 then stage 2, stage 2 then 1)
STEP_OPS = (("route_kernel", ("route+compact stage1", "route+compact stage2")),
            ("ema_tile_aggregate", ("dechunk stage2", "dechunk stage1")),
            ("cr_gram_prefix", ("coding_rate",)),
            ("topk_kernel", ("topk_select",)),
            ("gather_topk", ("gather",)),
            ("up_count", ("upsample_bins",)))
STEP_KERNELS = 48  # dispatches of one step (coding rate at d 512 in two halves: 2 x (gram + 1 diag + 11 panel))
MOPS_FLOPS = 512   # SQ_INSTS_VALU_MFMA_MOPS_* count MFMA work in units of 512 flops


def _dispatches(path: str):
    """(dispatch id, short kernel name, row) sorted by dispatch id (the order of enqueue)."""
    rows = list(csv.DictReader(open(path)))
    return sorted(((int(r["Dispatch_Id"]), _short(r["Kernel_Name"]), r) for r in rows), key=lambda t: t[0])


def _label_step(names):
    """Op label of every kernel of one step, from the kernels that open each op."""
    labels, seen, cur = [], {}, None
    for n in names:
        for head, ops in STEP_OPS:
            if n.startswith(head):
                i = seen.get(head, 0)
                cur = ops[min(i, len(ops) - 1)]
                seen[head] = i + 1
                break
        labels.append(cur)
    return labels


def _last_steps(path: str, nsteps: int, per_step: int = STEP_KERNELS):
    """The dispatches of the last `nsteps` steps, grouped per step: [(kernel, op, row), ...]."""
    ds = _dispatches(path)
    ids = sorted({d for d, _, _ in ds})
    keep = set(ids[-per_step * nsteps:])
    rows = [(d, n, r) for d, n, r in ds if d in keep]
    # a counter file has one row per (dispatch, counter): merge them per dispatch
    per, order = {}, []
    for d, n, r in rows:
        if d not in per:
            per[d] = (n, {}, r)
            order.append(d)
        if "Counter_Name" in r:
            per[d][1][r["Counter_Name"]] = per[d][1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    steps = []
    for i in range(nsteps):
        ds_i = order[i * per_step:(i + 1) * per_step]
        names = [per[d][0] for d in ds_i]
        labels = _label_step(names)
        steps.append([(per[d][0], lab, per[d][1], per[d][2]) for d, lab in zip(ds_i, labels)])
    return steps


def step_kernels(a):
    """Per (op, kernel) table of one bench.py step: time from the kernel trace
    (mean over the traced steps), HBM bytes from FETCH_SIZE / WRITE_SIZE
    (calibrated by the copy), MFMA flops from SQ_INSTS_VALU_MFMA_MOPS_*."""
    tsteps = _last_steps(_one(a.trace, "*kernel_trace.csv"), a.trace_steps, a.step_kernels)
    dur = {}
    for st in tsteps:
        for n, lab, _, r in st:
            key = (lab, n)
            dur.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    per_step = a.trace_steps

    def counters(d, name):
        if not d:
            return {}
        out = {}
        for n, lab, c, _ in _last_steps(_one(d, "*counter_collection.csv"), 1, a.step_kernels)[0]:
            if name in c:
                out[(lab, n)] = out.get((lab, n), 0.0) + c[name]
        return out

    fs = a.copy_bytes / (counter_copy(a.copy_fetch, "FETCH_SIZE") * 1024) if a.copy_fetch else None
    wsc = a.copy_bytes / (counter_copy(a.copy_write, "WRITE_SIZE") * 1024) if a.copy_write else None
    fetch = counters(a.fetch, "FETCH_SIZE")
    write = counters(a.write, "WRITE_SIZE")
    mb = counters(a.mfma, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    mf = counters(a.mfma, "SQ_INSTS_VALU_MFMA_MOPS_F32")
    lines = [f"# rocprofv3 summary: {a.workload}", "", "Commands (run from the repository root on the GPU host):",
             "", "```", a.cmd, "```", "",
             f"One step = the last {a.step_kernels} dispatches of each run.  Time: mean over the last "
             f"{a.trace_steps} traced steps of each kernel's summed durations per step.  Bytes: "
             f"FETCH_SIZE x {fs:.3f} and WRITE_SIZE x {wsc:.3f} (KiB per dispatch, scaled by a "
             f"{a.copy_bytes}-byte device copy), summed per step.  MFMA: SQ_INSTS_VALU_MFMA_MOPS_BF16 / _F32 "
             f"x {MOPS_FLOPS} flops; fraction of the 2500 (bf16) and 157.3 (fp32) TFLOP/s dense peaks.",
             "", "| op | kernel | launches | us per step | read GB | written GB | GB/s | HBM frac | "
             "bf16 TFLOP/s | fp32 TFLOP/s | MFMA frac |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    block = []
    for key in sorted(dur, key=lambda k: [lab for _, lab in STEP_OPS for lab in lab].index(k[0])
                      if k[0] in [x for _, l in STEP_OPS for x in l] else 99):
        lab, n = key
        us = sum(dur[key]) / per_step
        launches = len(dur[key]) / per_step
        rd = fetch.get(key, float("nan")) * 1024 * fs / 1e9 if fs else float("nan")
        wr = write.get(key, float("nan")) * 1024 * wsc / 1e9 if wsc else float("nan")
        gbs = (rd + wr) / (us * 1e-6)
        bft = mb.get(key, 0.0) * MOPS_FLOPS / (us * 1e-6) / 1e12
        f3t = mf.get(key, 0.0) * MOPS_FLOPS / (us * 1e-6) / 1e12
        mfrac = bft / 2500.0 + f3t / 157.3
        lines.append(f"| {lab} | {n} | {launches:g} | {us:.1f} | {rd:.3f} | {wr:.3f} | {gbs:.0f} | "
                     f"{gbs / 8000:.3f} | {bft:.1f} | {f3t:.1f} | {mfrac:.3f} |")
        block.append({"op": lab, "kernel": n, "launches": launches, "us": round(us, 2), "read_GB": round(rd, 4),
                      "write_GB": round(wr, 4), "GBps": round(gbs), "bf16_TFLOPs": round(bft, 1),
                      "fp32_TFLOPs": round(f3t, 1), "mfma_frac": round(mfrac, 4)})
    lines += ["", "```json", json.dumps({"step_kernels": block}), "```", ""]
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def step_timeline(a):
    """Start and end of every kernel of the last traced step, per HIP queue
    (stream), relative to the step's first kernel: how the streams of a
    scheduled step overlap.  The step starts at its first Gram-prefix kernel."""
    rows = list(csv.DictReader(open(_one(a.trace, "*kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    heads = [i for i, r in enumerate(rows) if _short(r["Kernel_Name"]).startswith("cr_gram_prefix")]
    if len(heads) < 2:
        raise ValueError(f"no whole step in {a.trace}")
    t0 = int(rows[heads[-2]]["Start_Timestamp"])  # the coding rate's two halves open the last step
    # with the steps overlapped, kernels of the step before may still run at its start
    step = [r for r in rows[:heads[-2]] if int(r["End_Timestamp"]) > t0] + rows[heads[-2]:]
    end = max(int(r["End_Timestamp"]) for r in step)
    lines = [f"# rocprofv3 summary: {a.workload}", "", "Commands (run from the repository root on the GPU host):",
             "", "```", a.cmd, "```", "",
             f"The last traced step: {len(step)} kernels over {(end - t0) / 1e3:.1f} us (kernel trace, so each "
             "kernel's span includes any time it shared the GPU with the other streams).  Times in us from the "
             "step's first kernel (negative: a kernel of the step before, still running); queue = the HIP queue "
             "(stream) it ran on.", "",
             "| start | end | us | queue | kernel |", "|---|---|---|---|---|"]
    for r in step:
        s0 = (int(r["Start_Timestamp"]) - t0) / 1e3
        s1 = (int(r["End_Timestamp"]) - t0) / 1e3
        lines.append(f"| {s0:.1f} | {s1:.1f} | {s1 - s0:.1f} | {r['Queue_Id']} | {_short(r['Kernel_Name'])} |")
    lines.append("")
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--op", required=True, choices=sorted(OPS) + ["step", "step-kernels", "step-timeline"])
    ap.add_argument("--mfma", help="--pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 ... run")
    ap.add_argument("--trace-steps", type=int, default=3, help="steps in the kernel-trace run (step-kernels)")
    ap.add_argument("--step-kernels", type=int, default=STEP_KERNELS, help="dispatches per step (step-kernels)")
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--last", type=int, default=0,
                    help="summarise the last N calls (the profiled steps); default: all but the first")
    ap.add_argument("--parts", type=int, default=1,
                    help="streams one call of the op runs on (first kernels per call)")
    ap.add_argument("--cmd", required=True, help="the full commands that produced the runs")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.op == "step-timeline":
        step_timeline(a)
        return
    if a.op == "step-kernels":
        step_kernels(a)
        return
    if a.op == "step":
        step_summary(a.trace, a.cmd, a.workload, a.out)
        return

    calls = trace_calls(a.op, a.trace, a.parts)
    if a.last > 0:
        timed = calls[-a.last:]  # bench.py's set-up may call the op's kernels more than once
    else:
        timed = calls[1:] if len(calls) > 1 else calls  # the first call is bench.py's set-up pass
    per_kernel = {}
    for c in timed:
        for r in c:
            per_kernel.setdefault(_short(r["Kernel_Name"]), []).append(
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    call_ns = [sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in c) for c in timed]
    span_ns = [max(int(r["End_Timestamp"]) for r in c) - min(int(r["Start_Timestamp"]) for r in c) for c in timed]

    lines = [f"# rocprofv3 summary: {a.op}, {a.workload}", "", "Commands (run from the repository root on the GPU host):", "",
             "```", a.cmd, "```", "",
             f"Calls profiled: {len(timed)} (the last ones of the run), each on {a.parts} stream(s).  "
             f"Time per call from its first kernel's start to its last kernel's end: "
             f"{statistics.mean(span_ns) / 1e3:.1f} us; sum of its kernels' durations "
             f"{statistics.mean(call_ns) / 1e3:.1f} us (more than the span where streams overlap).", "",
             "| kernel | launches per call | avg us | total us per call |", "|---|---|---|---|"]
    for k, v in sorted(per_kernel.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {k} | {len(v) / len(timed):g} | {statistics.mean(v) / 1e3:.1f} | "
                     f"{sum(v) / len(timed) / 1e3:.1f} |")
    block = {"op": a.op, "workload": a.workload, "us_per_call": round(statistics.mean(span_ns) / 1e3, 2),
             "kernel_us_per_call": round(statistics.mean(call_ns) / 1e3, 2), "parts": a.parts,
             "sources_sha256": sources_sha256(a.op)}
    if a.fetch and a.write and a.copy_fetch and a.copy_write:
        f_kib = counter_last_call(a.op, a.fetch, "FETCH_SIZE", a.parts)
        w_kib = counter_last_call(a.op, a.write, "WRITE_SIZE", a.parts)
        cf_kib = counter_copy(a.copy_fetch, "FETCH_SIZE")
        cw_kib = counter_copy(a.copy_write, "WRITE_SIZE")
        f_scale = a.copy_bytes / (cf_kib * 1024)
        w_scale = a.copy_bytes / (cw_kib * 1024)
        fetch_b = f_kib * 1024 * f_scale
        write_b = w_kib * 1024 * w_scale
        lines += ["", "HBM traffic per call (FETCH_SIZE and WRITE_SIZE, KiB summed over the call's "
                  "dispatches, scaled by a device copy of known size):", "",
                  f"- copy of {a.copy_bytes} B: FETCH_SIZE {cf_kib:.0f} KiB (scale {f_scale:.3f}), "
                  f"WRITE_SIZE {cw_kib:.0f} KiB (scale {w_scale:.3f})",
                  f"- {a.op}: FETCH_SIZE {f_kib:.0f} KiB -> {fetch_b / 1e9:.3f} GB read; "
                  f"WRITE_SIZE {w_kib:.0f} KiB -> {write_b / 1e9:.3f} GB written"]
        block.update({"fetch_bytes_per_call": round(fetch_b), "write_bytes_per_call": round(write_b),
                      "hbm_bytes_per_call": round(fetch_b + write_b),
                      "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)})
    lines += ["", "```json", json.dumps(block), "```", ""]
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
