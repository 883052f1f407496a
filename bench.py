"""Throughput of the dynamic-chunking layer on one MI355X.

One step = one pass of the whole chunk layer over one batch of 32 byte
streams of 8192 bytes each:
  * H-Net two-stage hierarchy (32 event streams of 8192 bytes): route with the
    stage's 0.75 score quantile, compact, route + compact the stage-2 rows,
    EMA-dechunk stage 2 back to stage-1 length, EMA-dechunk stage 1 back to
    bytes (d_local 512, d_mid 768, bf16);
  * ByteFlow layer (32 x 8192 x 512): coding rate Delta R (d 512, eps^2 0.5),
    BOS + Top-(K-1) with K = 2048, gather of the K rows, 16-bin multi-linear
    upsample from d_global 1536 with the residual (bf16).
The random stand-ins around the layer (q/k projections, the stage-2 input
projection, the projection back to d_local, the global map g = z W_g) are
computed once before the timed region.  Inputs are resident in HBM when
timing starts.  value = 32 * 8192 byte positions / step time.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
BF16_MFMA_PEAK_TFLOPS = 2500.0
COPY_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--schedule", default="pipelined",
                    choices=["pipelined", "after_dr", "routes_with_dr", "with_dr", "serial"],
                    help="where the H-Net layer runs in a step: on a stream of its own beside Top-K, gather "
                         "and upsample (after_dr), the same with that stream joined back only after the last "
                         "step, so that it also runs beside the next step's Delta R (pipelined, the default), "
                         "beside Delta R (with_dr), its routing beside Delta R and its dechunks after it "
                         "(routes_with_dr), or every op on one stream in turn (serial); the others are timed "
                         "as well")
    ap.add_argument("--profile-op", default=None,
                    help="run only this op (or 'step': the whole step with its ops queued in turn; "
                         "'step-scheduled': the whole step in the --schedule order; 'copy': a 1 GiB device "
                         "copy) --steps times after set-up, untimed (for rocprofv3)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Workload:
    """Device-resident inputs, stand-ins, outputs and workspaces of one step."""

    def __init__(self):
        import torch
        import byte_level_lm_amd as B
        from synthdata import gen_hnet_two_stage, gen_byteflow_layer

        self.B = B
        self.torch = torch
        bf = torch.bfloat16
        dev = torch.device("cuda")
        t0 = time.time()
        hn = gen_hnet_two_stage(fixed_T=8192)
        bfl = gen_byteflow_layer()
        log(f"inputs generated in {time.time() - t0:.1f}s")
        self.hn, self.bfl = hn, bfl
        T = 8192
        self.nseq = 32
        self.N = int(hn["offsets"][-1])
        assert self.N == self.nseq * T
        # ---------------- H-Net
        self.off = torch.from_numpy(hn["offsets"]).to(dev)
        self.h1 = torch.from_numpy(hn["h"]).to(dev, bf)
        self.q1 = torch.from_numpy(hn["q"]).to(dev, bf)
        self.k1 = torch.from_numpy(hn["k"]).to(dev, bf)
        N = self.N
        self.p1 = torch.empty(N, device=dev)
        self.b1 = torch.empty(N, dtype=torch.uint8, device=dev)
        self.tau1 = torch.empty(1, device=dev)
        self.ws_route = torch.empty(B.route_workspace(N), dtype=torch.uint8, device=dev)
        self.ws_compact = torch.empty(B.compact_workspace(N), dtype=torch.uint8, device=dev)
        self.idx1 = torch.empty(N, dtype=torch.int32, device=dev)
        self.coff1 = torch.empty(self.nseq + 1, dtype=torch.int64, device=dev)
        self.z1 = torch.empty((N, 512), dtype=bf, device=dev)
        self.P1 = torch.empty(N, device=dev)
        self.st = torch.zeros(1, dtype=torch.int32, device=dev)
        # untimed first pass of stage 1 to size stage 2 and build its stand-in inputs
        self._stage1()
        torch.cuda.synchronize()
        self.M1 = int(self.coff1[-1].item())
        M1 = self.M1
        w_mid = torch.from_numpy(hn["w_mid"]).to(dev, torch.float32)
        wq2 = torch.from_numpy(hn["wq2"]).to(dev, torch.float32)
        wk2 = torch.from_numpy(hn["wk2"]).to(dev, torch.float32)
        self.x2 = (self.z1[:M1].float() @ w_mid).to(bf)
        self.q2 = (self.x2.float() @ wq2).to(bf)
        self.k2 = (self.x2.float() @ wk2).to(bf)
        self.p2 = torch.empty(M1, device=dev)
        self.b2 = torch.empty(M1, dtype=torch.uint8, device=dev)
        self.tau2 = torch.empty(1, device=dev)
        self.idx2 = torch.empty(M1, dtype=torch.int32, device=dev)
        self.coff2 = torch.empty(self.nseq + 1, dtype=torch.int64, device=dev)
        self.z2 = torch.empty((M1, 768), dtype=bf, device=dev)
        self.P2 = torch.empty(M1, device=dev)
        self.y2 = torch.empty((M1, 768), dtype=bf, device=dev)
        self.out1 = torch.empty((N, 512), dtype=bf, device=dev)
        self.ws_dechunk = torch.empty(B.dechunk_workspace(768), dtype=torch.uint8, device=dev)
        self._stage2()
        self._dechunk2()
        torch.cuda.synchronize()
        self.M2 = int(self.coff2[-1].item())
        w_back = torch.from_numpy(hn["w_back"]).to(dev, torch.float32)
        self.y1 = (self.y2.float() @ w_back).to(bf)  # stand-in projection back to d_local
        # ---------------- ByteFlow
        self.K, self.nbins = bfl["K"], bfl["nbins"]
        self.h4 = torch.from_numpy(bfl["h"]).to(dev, bf)
        self.off4 = torch.arange(self.nseq + 1, dtype=torch.int64, device=dev) * T
        self.dR = torch.empty((self.nseq, T), device=dev)
        # the coding rate runs its batch as two halves on two streams of ours
        # (forked from and joined back to the current stream by two events)
        self.cr_stream2 = torch.cuda.Stream()
        self.cr_fork, self.cr_join = torch.cuda.Event(), torch.cuda.Event()
        # the H-Net layer shares no buffer with the ByteFlow chain: in a step it
        # runs on a stream of its own, forked from and joined back to the
        # current stream
        self.h_stream = torch.cuda.Stream()
        self.h_fork, self.h_join = torch.cuda.Event(), torch.cuda.Event()
        self.ws_cr = torch.empty(B.coding_rate_workspace(self.nseq, T, 512), dtype=torch.uint8, device=dev)
        self.idx4 = torch.empty((self.nseq, self.K), dtype=torch.int32, device=dev)
        self.z4 = torch.empty((self.nseq * self.K, 512), dtype=bf, device=dev)
        self.W = torch.from_numpy(bfl["w_bin"]).to(dev, bf)
        self.s4 = torch.empty_like(self.h4)
        self.ws_up = torch.empty(B.upsample_workspace(self.nseq, T, self.K, 1536, 512, self.nbins),
                                 dtype=torch.uint8, device=dev)
        self._coding_rate(); self._topk(); self._gather()
        torch.cuda.synchronize()
        w_g = torch.from_numpy(bfl["w_g"]).to(dev, torch.float32)
        self.g4 = (self.z4.float() @ w_g).to(bf).view(self.nseq, self.K, 1536)  # global stand-in
        self._upsample()
        torch.cuda.synchronize()
        # ---------------- next rows, timed outside the step
        # cosine-score chunker: stand-in routing projections of ByteFlow's h (untimed)
        h4f = self.h4.view(-1, 512).float()
        self.q4 = (h4f @ torch.from_numpy(bfl["wq"]).to(dev, torch.float32)).to(bf)
        self.k4 = (h4f @ torch.from_numpy(bfl["wk"]).to(dev, torch.float32)).to(bf)
        del h4f
        self.p4 = torch.empty(N, device=dev)
        self.b4 = torch.empty(N, dtype=torch.uint8, device=dev)
        self.idx5 = torch.empty((self.nseq, self.K), dtype=torch.int32, device=dev)
        self.mask5 = torch.empty((self.nseq, T), dtype=torch.uint8, device=dev)
        self._cosine_chunker()
        # EMA dechunk backward of stage 1: a seeded stand-in output gradient (untimed)
        gen = torch.Generator(device=dev)
        gen.manual_seed(20260005)
        self.dout1 = torch.randn((N, 512), generator=gen, device=dev).to(bf)
        self.dz1 = torch.empty((self.M1, 512), dtype=bf, device=dev)
        self.dP1 = torch.empty(self.M1, device=dev)
        self.ws_dbwd = torch.empty(B.dechunk_ema_backward_workspace(512, self.M1), dtype=torch.uint8, device=dev)
        self._dechunk1_backward()
        # stage-1 routing straight from h (projections inside the kernel)
        self.wq1 = torch.from_numpy(hn["wq"]).to(dev, bf)
        self.wk1 = torch.from_numpy(hn["wk"]).to(dev, bf)
        self.pf1 = torch.empty(N, device=dev)
        self.bf1 = torch.empty(N, dtype=torch.uint8, device=dev)
        self.tauf1 = torch.empty(1, device=dev)
        self.ws_routef = torch.empty(B.route_workspace(N), dtype=torch.uint8, device=dev)
        # the unfused reference for it: the two projections through torch's
        # library GEMM into q and k, then bllm_route on them
        self.ql1 = torch.empty((N, 512), dtype=bf, device=dev)
        self.kl1 = torch.empty((N, 512), dtype=bf, device=dev)
        # streaming chunker: the same byte streams arriving in windows of 1024
        # bytes, each its own dense buffer; the carried matrix is updated in place
        self.win = 1024
        self.Kw = self.K * self.win // T
        self.h4w = [self.h4[:, i * self.win:(i + 1) * self.win].contiguous() for i in range(T // self.win)]
        self.state4 = torch.empty((self.nseq, 512, 512), device=dev)
        self.dRw = torch.empty((self.nseq, self.win), device=dev)
        self.idxw = torch.empty((T // self.win, self.nseq, self.Kw), dtype=torch.int32, device=dev)
        self.maskw = torch.empty((T // self.win, self.nseq, self.win), dtype=torch.uint8, device=dev)
        self.ws_crw = torch.empty(B.coding_rate_workspace(self.nseq, self.win, 512), dtype=torch.uint8, device=dev)
        self._streaming_chunker()
        self._route_fused1()
        self._route_library1()
        torch.cuda.synchronize()
        log(f"setup done: M1={self.M1} ({self.M1 / N:.3f} N), M2={self.M2} ({self.M2 / N:.3f} N)")

    # ------------------------------------------------------------ ops of one step
    def _stage1(self):
        B = self.B
        B.route(self.q1, self.k1, self.off, quantile=0.75, p_out=self.p1, b_out=self.b1, tau_out=self.tau1,
                status=self.st, ws=self.ws_route)
        B.compact(self.b1, self.off, rows=self.h1, p=self.p1, capacity=self.N, idx_out=self.idx1,
                  chunk_offsets_out=self.coff1, rows_out=self.z1, P_out=self.P1, status=self.st,
                  ws=self.ws_compact)

    def _stage2(self):
        B = self.B
        B.route(self.q2, self.k2, self.coff1, quantile=0.75, p_out=self.p2, b_out=self.b2,
                tau_out=self.tau2, status=self.st, ws=self.ws_route)
        B.compact(self.b2, self.coff1, rows=self.x2, p=self.p2, capacity=self.M1, idx_out=self.idx2,
                  chunk_offsets_out=self.coff2, rows_out=self.z2, P_out=self.P2, status=self.st,
                  ws=self.ws_compact)

    def _dechunk2(self):
        self.B.dechunk_ema(self.z2, self.P2, self.idx2, self.coff2, self.coff1, self.M1, out=self.y2,
                           ws=self.ws_dechunk)

    def _dechunk1(self):
        self.B.dechunk_ema(self.y1, self.P1, self.idx1, self.coff1, self.off, self.N, out=self.out1,
                           ws=self.ws_dechunk)

    def _coding_rate(self):
        self.B.coding_rate_split(self.h4, 0.5, self.cr_stream2, self.cr_fork, self.cr_join, dR_out=self.dR,
                                 status=self.st, ws=self.ws_cr)

    def _topk(self):
        self.B.topk_select(self.dR, self.K, idx_out=self.idx4, status=self.st, want_mask=False)

    def _gather(self):
        self.B.gather_topk(self.h4, self.idx4, z_out=self.z4.view(self.nseq, self.K, 512))

    def _upsample(self):
        self.B.upsample_bins(self.g4, self.W, self.idx4, self.h4, self.nbins, s_out=self.s4, ws=self.ws_up)

    def _cosine_chunker(self):
        self.B.route(self.q4, self.k4, self.off4, threshold=0.5, p_out=self.p4, b_out=self.b4)
        self.B.topk_select(self.p4.view(self.nseq, -1), self.K, idx_out=self.idx5, mask_out=self.mask5,
                           status=self.st)

    def _streaming_chunker(self):
        for i, hw in enumerate(self.h4w):
            self.B.coding_rate_stream(hw, 0.5, None if i == 0 else self.state4, state_out=self.state4,
                                      dR_out=self.dRw, status=self.st, ws=self.ws_crw)
            self.B.topk_select_window(self.dRw, self.Kw, i == 0, idx_out=self.idxw[i], mask_out=self.maskw[i],
                                      status=self.st)

    def _dechunk1_backward(self):
        self.B.dechunk_ema_backward(self.y1, self.P1, self.dout1, self.idx1, self.coff1, self.off,
                                    dz_out=self.dz1, dP_out=self.dP1, ws=self.ws_dbwd, max_chunks=self.M1)

    def _route_fused1(self):
        self.B.route_fused(self.h1, self.wq1, self.wk1, self.off, quantile=0.75, p_out=self.pf1, b_out=self.bf1,
                           tau_out=self.tauf1, ws=self.ws_routef)

    def _route_library1(self):
        torch = self.torch
        torch.matmul(self.h1, self.wq1, out=self.ql1)
        torch.matmul(self.h1, self.wk1, out=self.kl1)
        self.B.route(self.ql1, self.kl1, self.off, quantile=0.75, p_out=self.pf1, b_out=self.bf1,
                     tau_out=self.tauf1, ws=self.ws_routef)

    def next_ops(self):
        """Rows past the hot path (fused projection, cosine chunker, EMA backward, streaming
        chunker), timed on their own, and the unfused reference of the fused projection."""
        return [("cosine_chunker", self._cosine_chunker), ("dechunk_backward stage1", self._dechunk1_backward),
                ("route_fused stage1", self._route_fused1),
                ("library GEMM + route stage1", self._route_library1),
                ("streaming_chunker", self._streaming_chunker)]

    def next_algorithmic(self):
        N, M1, nseq, K = self.N, self.M1, self.nseq, self.K
        e = 2
        return {"cosine_chunker": dict(bytes=N * (2 * 512 * e + 4 + 1) + N * 4 + N + nseq * K * 4),
                # dout read once, z and P read, dz and dP written
                "dechunk_backward stage1": dict(bytes=N * 512 * e + M1 * (2 * 512 * e + 4 + 4 + 4)),
                # h read once, Wq and Wk, p and b written; q = h Wq and k = h Wk on bf16 MFMA
                "route_fused stage1": dict(bytes=N * (512 * e + 5) + 2 * 512 * 512 * e,
                                           flops=2 * N * 512 * 1024),
                # the same work unfused: q and k written by the GEMMs and read back by the route
                "library GEMM + route stage1": dict(bytes=N * (512 * e + 5) + 2 * 512 * 512 * e
                                                    + 2 * 2 * N * 512 * e, flops=2 * N * 512 * 1024),
                # every window: h read, Delta R written, the carried matrix read and written, the
                # local selection; the same 3 T d^2 MFMA count as the whole-sequence coding rate
                "streaming_chunker": dict(flops=3 * N * 512 * 512, peak_tflops=FP32_MFMA_PEAK_TFLOPS,
                                          bytes=N * (512 * e + 4 + 4 + 1) + nseq * K * 4
                                          + len(self.h4w) * nseq * 512 * 512 * 4 * 2)}

    def ops(self):
        return [("route+compact stage1", self._stage1), ("route+compact stage2", self._stage2),
                ("dechunk stage2", self._dechunk2), ("dechunk stage1", self._dechunk1),
                ("coding_rate", self._coding_rate), ("topk_select", self._topk),
                ("gather", self._gather), ("upsample_bins", self._upsample)]

    def hnet_ops(self):
        return self.ops()[:4]

    def byteflow_ops(self):
        return self.ops()[4:]

    def step(self, dom=None, schedule="after_dr", last=True):
        """One pass of the whole path.  The H-Net layer (stage 1 and 2 routing
        and compaction, both dechunks) and the ByteFlow chain (Delta R, Top-K,
        gather, upsample) take different inputs and share no buffer.
        schedule "serial" queues every op on the current stream in turn; the
        others run the H-Net layer on a stream of its own, forked from the
        current stream at the start of the step ("with_dr") or once Delta R is
        queued, beside Top-K, gather and upsample ("after_dr"), or its routing
        and compaction beside Delta R and its dechunks after it
        ("routes_with_dr"), and joined back before the step ends.
        "pipelined" is "after_dr" across steps: the H-Net stream is joined
        back only after the last of a run of steps (last=True), so a step's
        ByteFlow chain, from Delta R on, runs beside the previous step's
        H-Net dechunks (the streams' own order keeps each layer's steps in
        sequence; the two layers share no buffer).  dom: a pair of events
        recorded around the coding rate on the current stream."""
        torch = self.torch
        cur = torch.cuda.current_stream()
        join = last or schedule != "pipelined"
        if schedule == "pipelined":
            schedule = "after_dr"

        def fork_hnet(part=slice(None)):
            self.h_fork.record(cur)
            self.h_stream.wait_event(self.h_fork)
            with torch.cuda.stream(self.h_stream):
                for _, f in self.hnet_ops()[part]:
                    f()
                self.h_join.record(self.h_stream)

        if schedule == "with_dr":
            fork_hnet()
        elif schedule == "routes_with_dr":
            fork_hnet(slice(0, 2))  # both stages' routing and compaction
        for name, f in (self.ops() if schedule == "serial" else self.byteflow_ops()):
            if dom is not None and name == "coding_rate":
                dom[0].record(cur)
                f()
                dom[1].record(cur)
            else:
                f()
            if name == "coding_rate" and schedule == "after_dr":
                fork_hnet()
            elif name == "coding_rate" and schedule == "routes_with_dr":
                fork_hnet(slice(2, 4))  # the two dechunks, after the routing on the same stream
        if schedule != "serial" and join:
            cur.wait_event(self.h_join)

    # ------------------------------------------------------------ algorithmic work
    def algorithmic(self):
        """Algorithmic HBM bytes / MFMA flops per op (what the method must touch)."""
        N, M1, M2, nseq, K = self.N, self.M1, self.M2, self.nseq, self.K
        e = 2
        idx = self.idx4.cpu().numpy()
        T = 8192
        items = 0
        for s in range(nseq):
            L = np.diff(np.concatenate([idx[s], [T]]))
            items += int(np.minimum(L, self.nbins).sum())
        self.up_items = items
        return {
            "route+compact stage1": dict(bytes=N * (2 * 512 * e + 4 + 1) + N + M1 * (4 + 4 + 4 + 2 * 512 * e)),
            "route+compact stage2": dict(bytes=M1 * (2 * 768 * e + 4 + 1) + M1 + M2 * (4 + 4 + 4 + 2 * 768 * e)),
            "dechunk stage2": dict(bytes=M2 * (768 * e + 8) + M1 * 768 * e),
            "dechunk stage1": dict(bytes=M1 * (512 * e + 8) + N * 512 * e),
            "coding_rate": dict(flops=3 * T * 512 * 512 * nseq, bytes=N * 512 * e + N * 4,
                                peak_tflops=FP32_MFMA_PEAK_TFLOPS),
            "topk_select": dict(bytes=N * 4 + nseq * K * 4),
            "gather": dict(bytes=nseq * K * (4 + 2 * 512 * e)),
            "upsample_bins": dict(flops=2 * 1536 * 512 * items, bytes=2 * N * 512 * e + nseq * K * 1536 * e),
        }


def time_fn(torch, f, reps=7):
    """Median of `reps` timed calls of f (HIP events on torch's current stream)."""
    f()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        f()
        ev1.record()
        torch.cuda.synchronize()
        ts.append(ev0.elapsed_time(ev1))
    return float(np.median(ts))


def other_workloads(B, torch):
    """The other two full-size workloads, each timed on its own (median of 7
    calls of the whole chain, inputs resident): the ByteGen-style event
    streams through one H-Net stage (16 ragged streams of 32 x U{32..256}
    events, d 512 bf16, threshold 0.5: route, compact, EMA dechunk) and the
    fp32 coding-rate chunker (8 x 8192 x 256, K 2048: Delta R, Top-K,
    gather)."""
    from synthdata import gen_event_streams, gen_coding_rate_fp32
    bf = torch.bfloat16
    out = {}
    # ---- event streams, one H-Net stage
    c = gen_event_streams()
    off = torch.from_numpy(c["offsets"]).cuda()
    N = int(c["offsets"][-1])
    nseq = len(c["offsets"]) - 1
    q = torch.from_numpy(c["q"]).to("cuda", bf)
    k = torch.from_numpy(c["k"]).to("cuda", bf)
    h = torch.from_numpy(c["h"]).to("cuda", bf)
    p = torch.empty(N, device="cuda")
    b = torch.empty(N, dtype=torch.uint8, device="cuda")
    idx = torch.empty(N, dtype=torch.int32, device="cuda")
    coff = torch.empty(nseq + 1, dtype=torch.int64, device="cuda")
    z = torch.empty((N, 512), dtype=bf, device="cuda")
    P = torch.empty(N, device="cuda")
    o = torch.empty((N, 512), dtype=bf, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    wsc = torch.empty(B.compact_workspace(N), dtype=torch.uint8, device="cuda")
    wsd = torch.empty(B.dechunk_workspace(512), dtype=torch.uint8, device="cuda")

    def c1():
        B.route(q, k, off, threshold=0.5, p_out=p, b_out=b, status=st)
        B.compact(b, off, rows=h, p=p, capacity=N, idx_out=idx, chunk_offsets_out=coff, rows_out=z, P_out=P,
                  status=st, ws=wsc)
        B.dechunk_ema(z, P, idx, coff, off, N, out=o, ws=wsd, max_chunks=N)

    ms = time_fn(torch, c1)
    M = int(coff[-1].item())
    e = 2
    alg = N * (2 * 512 * e + 5) + N + M * (4 + 4 + 4 + 2 * 512 * e) + M * (512 * e + 8) + N * 512 * e
    out["event_streams_hnet_stage_B16_ragged"] = {
        "ms": round(ms, 4), "bytes_per_s": N / (ms * 1e-3), "positions": N, "boundaries": M,
        "hbm_GBps": round(alg / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "status_word": int(st.item())}
    del q, k, h, z, o
    # ---- fp32 coding-rate chunker
    c = gen_coding_rate_fp32()
    ns, T, d, K = c["nseq"], c["T"], c["d"], c["K"]
    hf = torch.from_numpy(c["h"]).cuda()
    dR = torch.empty((ns, T), device="cuda")
    ws = torch.empty(B.coding_rate_workspace(ns, T, d), dtype=torch.uint8, device="cuda")
    sel = torch.empty((ns, K), dtype=torch.int32, device="cuda")
    mask = torch.empty((ns, T), dtype=torch.uint8, device="cuda")
    off3 = torch.arange(ns + 1, dtype=torch.int64, device="cuda") * T
    gidx = torch.empty(ns * K, dtype=torch.int32, device="cuda")
    co3 = torch.empty(ns + 1, dtype=torch.int64, device="cuda")
    z3 = torch.empty((ns * K, d), device="cuda")
    wsc3 = torch.empty(B.compact_workspace(ns * T), dtype=torch.uint8, device="cuda")
    st.zero_()

    def c3_dr():
        B.coding_rate(hf, c["eps2"], dR_out=dR, status=st, ws=ws)

    def c3():
        c3_dr()
        B.topk_select(dR, K, idx_out=sel, mask_out=mask, status=st)
        B.compact(mask.view(-1), off3, rows=hf.view(-1, d), capacity=ns * K, idx_out=gidx, chunk_offsets_out=co3,
                  rows_out=z3, status=st, ws=wsc3)

    ms = time_fn(torch, c3)
    ms_dr = time_fn(torch, c3_dr)
    flops = 3 * T * d * d * ns
    out["coding_rate_fp32_B8_T8192_d256_K2048"] = {
        "ms": round(ms, 4), "bytes_per_s": ns * T / (ms * 1e-3), "coding_rate_ms": round(ms_dr, 4),
        "coding_rate_TFLOPs": round(flops / (ms_dr * 1e-3) / 1e12, 2),
        "coding_rate_fp32_mfma_frac": round(flops / (ms_dr * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
        "status_word": int(st.item())}
    return out


def coding_rate_traffic():
    """HBM bytes per bllm_coding_rate call from the committed rocprofv3 counter
    summary, or None when it is missing or its sources have changed since."""
    import re
    from byte_level_lm_amd.profsum import sources_sha256
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "coding_rate_bf16_32x8192x512.md")
    try:
        text = open(path).read()
        block = json.loads(re.findall(r"```json\n(.*?)\n```", text, re.S)[-1])
    except (OSError, IndexError, ValueError):
        return None
    if block.get("sources_sha256") != sources_sha256("coding_rate") or "hbm_bytes_per_call" not in block:
        return None
    return block["hbm_bytes_per_call"]


def op_rates(a, t):
    """Time of one op with its algorithmic HBM rate and MFMA rate, each also as
    a fraction of MI355X's peak (8 TB/s; dense MFMA of the op's arithmetic type)."""
    d = {"ms": round(t, 4)}
    if "bytes" in a:
        gbps = a["bytes"] / (t * 1e-3) / 1e9
        d["hbm_GBps"] = round(gbps, 1)
        d["hbm_frac"] = round(gbps / HBM_PEAK_GBS, 4)
    if "flops" in a:
        tf = a["flops"] / (t * 1e-3) / 1e12
        peak = a.get("peak_tflops", BF16_MFMA_PEAK_TFLOPS)
        d["TFLOPs"] = round(tf, 2)
        d["mfma_frac"] = round(tf / peak, 4)
        d["mfma_peak"] = peak
    return d


def op_ideal_ms(name, a):
    """Ideal time of one op at MI355X's peaks: max(algorithmic HBM bytes / 8 TB/s,
    algorithmic flops / the peak of the narrowest type that keeps the op's
    accuracy).  The coding rate's Gram (2 of its 3 T d^2 flops per sequence)
    is exact in bf16, its solves need fp32; the upsample is a bf16 GEMM."""
    t_hbm = a.get("bytes", 0) / (HBM_PEAK_GBS * 1e9)
    f = a.get("flops", 0)
    if name == "coding_rate":
        t_mfma = 2 * f / 3 / (BF16_MFMA_PEAK_TFLOPS * 1e12) + f / 3 / (FP32_MFMA_PEAK_TFLOPS * 1e12)
    else:
        t_mfma = f / (a.get("peak_tflops", BF16_MFMA_PEAK_TFLOPS) * 1e12)
    return max(t_hbm, t_mfma) * 1e3


SCHEDULES = {"pipelined": "H-Net layer on a stream of its own beside Top-K, gather and upsample and, across "
                          "steps, beside the next step's Delta R (joined back after the last step)",
             "after_dr": "H-Net layer on a stream of its own beside Top-K, gather and upsample",
             "routes_with_dr": "H-Net routing and compaction (both stages) on a stream of its own beside Delta R, "
                               "its two dechunks on that stream beside Top-K, gather and upsample",
             "with_dr": "H-Net layer on a stream of its own beside Delta R",
             "serial": "every op on one stream in turn"}


def step_roofline(alg, ms):
    """% roofline of a whole step: the sum of the ops' ideal times over the measured step time."""
    ideal = sum(op_ideal_ms(n, a) for n, a in alg.items())
    return {"ideal_ms": round(ideal, 4), "measured_ms": round(ms, 4), "frac": round(ideal / ms, 4)}


MALL_FLUSH_BYTES = 512 << 20  # twice the 256 MB Infinity Cache


def time_ops(wl, reps=7, ops=None):
    """Median duration of each op (HIP events on the stream the kernels run
    on), each call preceded by a write of 512 MB so that no op finds its
    inputs in the 256 MB Infinity Cache from its previous call."""
    torch = wl.torch
    flush = torch.empty(MALL_FLUSH_BYTES // 4, device="cuda")
    res = {}
    for name, f in (wl.ops() if ops is None else ops):
        f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            flush.fill_(1.0)
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record()
            f()
            ev1.record()
            torch.cuda.synchronize()
            ts.append(ev0.elapsed_time(ev1))
        res[name] = float(np.median(ts))
    del flush
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_sample(args):
    """The oracle on one stream of each workload (stream index i), one BLAS
    thread: per-byte seconds of the H-Net layer, Delta R, Top-K + gather and
    the upsample, and the seconds spent."""
    i, dR_i = args
    from threadpoolctl import threadpool_limits
    import oracle
    from synthdata import gen_stage2_inputs, gen_stage2_backproj, gen_global_standin

    hn, bfl = _POOL_DATA["hn"], _POOL_DATA["bfl"]
    T = 8192
    with threadpool_limits(limits=1):
        # H-Net two-stage layer on stream i (8192 bytes)
        t0 = time.perf_counter()
        off = np.array([0, T], np.int64)
        q, k, h = hn["q"][i * T:(i + 1) * T], hn["k"][i * T:(i + 1) * T], hn["h"][i * T:(i + 1) * T]
        p1 = oracle.route(q, k, off)
        tau1 = oracle.stage_quantile(p1, 0.75)
        b1 = oracle.boundary_mask(p1, tau1)
        i1, co1, z1, P1 = oracle.compact(b1, p1, h, off)
        s2 = gen_stage2_inputs(z1, hn)
        t_standin = time.perf_counter()
        p2 = oracle.route(s2["q2"], s2["k2"], co1)
        t_standin = time.perf_counter() - t_standin
        tau2 = oracle.stage_quantile(p2, 0.75)
        b2 = oracle.boundary_mask(p2, tau2)
        i2, co2, z2, P2 = oracle.compact(b2, p2, s2["x2"], co1)
        y2 = oracle.dechunk_ema(z2, P2, i2, co2, co1)
        y1 = gen_stage2_backproj(y2, hn)
        oracle.dechunk_ema(y1, P1, i1, co1, off)
        t_hnet = time.perf_counter() - t0
        # ByteFlow: Delta R on the first npos positions of stream i
        npos = 3072  # the per-position cost (one d x d Cholesky) does not depend on t
        t0 = time.perf_counter()
        oracle.coding_rate_at(bfl["h"][i].astype(np.float64), 0.5, np.arange(npos))
        t_dr = time.perf_counter() - t0
        t0 = time.perf_counter()
        sel = oracle.topk_select(dR_i[None], _POOL_DATA["K"])
        z = oracle.gather(bfl["h"][i:i + 1], sel)
        t_topk = time.perf_counter() - t0
        g = gen_global_standin(z, bfl)
        nup = 2048
        t0 = time.perf_counter()
        # upsample of the first nup positions of the stream (same per-position work)
        cmap, bins = oracle.chunk_bins(sel[0], T, bfl["nbins"])
        hh = bfl["h"][i].astype(np.float64)
        W = bfl["w_bin"].astype(np.float64)
        gg = g[0].astype(np.float64)
        for t in range(nup):
            _ = hh[t] + gg[cmap[t]] @ W[bins[t]]
        t_up = time.perf_counter() - t0
    return dict(sec_per_byte=t_hnet / T + t_dr / npos + t_topk / T + t_up / nup,
                secs=(t_hnet, t_dr, t_topk, t_up), npos=npos, nup=nup)


_POOL_DATA = {}


def cpu_baseline(wl):
    """The oracle, as it stands, on a bounded sample of the same workload:
    the same per-stream sample (H-Net layer, Delta R at 3072 positions, Top-K
    + gather, 2048 upsampled positions) once on one core, then on one stream
    per worker process over all the host cores this process may use (at most
    16, the GPU's share of the box), each worker on its own stream."""
    import multiprocessing as mp
    T = 8192
    _POOL_DATA.update(hn=wl.hn, bfl=wl.bfl, K=wl.K)
    dR = wl.dR.cpu().numpy()
    one = _oracle_sample((0, dR[0]))
    ncores = max(1, min(16, len(os.sched_getaffinity(0)), wl.nseq))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(ncores) as pool:
        res = pool.map(_oracle_sample, [(i, dR[i]) for i in range(ncores)])
    wall = time.perf_counter() - t0
    # every worker covered one stream's worth of bytes at its own per-byte cost
    bytes_per_s = sum(1.0 / r["sec_per_byte"] for r in res)
    t_hnet, t_dr, t_topk, t_up = one["secs"]
    return {
        "value": bytes_per_s,
        "unit": "bytes/s",
        "cores": ncores,
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "one_core_value": 1.0 / one["sec_per_byte"],
        "sample": (f"oracle fp64, one BLAS thread per process, {ncores} processes (one stream of the "
                   f"32 each; {wall:.1f}s wall) after one process alone: per stream the H-Net two-stage "
                   f"layer ({T} B, {t_hnet:.1f}s alone incl. stand-ins), Delta R at the first "
                   f"{one['npos']} positions ({t_dr:.1f}s), Top-K + gather ({t_topk:.2f}s), upsample of "
                   f"{one['nup']} positions ({t_up:.1f}s); per-byte costs summed per stream, the "
                   f"streams' rates added"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.profile_op == "copy":
        # plain device copy of a known size: the calibration for the HBM byte counters
        src = torch.ones(COPY_BYTES // 4, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("profiled copy of", COPY_BYTES, "bytes,", args.steps, "launches")
        return
    wl = Workload()
    if args.profile_op:
        # the whole step with its ops queued in turn, so that each kernel's time
        # under the profiler is its own and not shared with the H-Net stream
        if args.profile_op == "step":
            f = lambda last: wl.step(schedule="serial")
        elif args.profile_op == "step-scheduled":
            f = lambda last: wl.step(schedule=args.schedule, last=last)  # the streams' overlap as timed
        else:
            op = dict(wl.ops() + wl.next_ops())[args.profile_op]
            f = lambda last: op()
        for i in range(args.steps):
            f(i == args.steps - 1)
        torch.cuda.synchronize()
        log("profiled", args.profile_op, args.steps, "launches")
        return
    for _ in range(args.warmup):
        for sch in SCHEDULES:
            wl.step(schedule=sch)
    torch.cuda.synchronize()
    log("warmup done")
    # the dominant op is bracketed by events of its own on the current stream
    # inside the timed steps (the coding rate's second stream is joined back
    # to it before the closing event)
    dom_name = "coding_rate"

    def timed_steps(schedule):
        dom_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
        t0 = time.perf_counter()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(args.steps):
            wl.step(dom=dom_ev[i], schedule=schedule, last=i == args.steps - 1)
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = ev0.elapsed_time(ev1) / args.steps
        dom_ms = sum(a.elapsed_time(b) for a, b in dom_ev) / args.steps
        log(f"timed {args.steps} steps ({schedule}): {ms:.3f} ms/step (wall {wall:.2f}s)")
        return ms, dom_ms

    ms, dom_ms = timed_steps(args.schedule)
    others = {sch: timed_steps(sch) for sch in SCHEDULES if sch != args.schedule}
    per_op = time_ops(wl)
    alg = wl.algorithmic()
    breakdown = {name: op_rates(alg[name], t) for name, t in per_op.items()}
    cr = alg["coding_rate"]
    # The 3 T d^2 algorithmic flops of Delta R: the Gram's 2 T d^2 are exact in
    # bf16 (priced at the bf16 MFMA peak), the solves' T d^2 need fp32 (fp32
    # MFMA peak).  The op's peak is the blend of the two, flops / ideal time,
    # so that achieved / peak = ideal time / measured time.
    ideal_ms = op_ideal_ms("coding_rate", cr)
    blended_peak = cr["flops"] / (ideal_ms * 1e-3) / 1e12
    roof = {
        "kernel": ("one bllm_coding_rate_split call (32 x 8192 x 512 bf16, two halves of 16 sequences on two "
                   "streams): per half cr_gram_prefix_bf16 + 1 cr_diag + 11 cr_panel (each factoring the next "
                   "diagonal tile); Gram on bf16 MFMA, "
                   "factorization in fp32 arithmetic (strip products as exact three-part bf16 MFMA, diagonal and "
                   "TRSM on fp32 MFMA)"),
        "bound": "mfma",
        "achieved": round(cr["flops"] / (dom_ms * 1e-3) / 1e12, 3),
        "peak": round(blended_peak, 2),
        "peak_basis": "2/3 of the flops at 2500 TFLOP/s (bf16 Gram), 1/3 at 157.3 TFLOP/s (fp32 solves)",
        "unit": "TFLOP/s",
        "traffic": coding_rate_traffic(),
    }
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["op_ms"] = round(dom_ms, 4)
    if "after_dr" in others:
        # the same op's live time in the steps where it has the chip to itself
        roof["op_ms_alone"] = round(others["after_dr"][1], 4)
        roof["frac_alone"] = round(ideal_ms / others["after_dr"][1], 4)
    roof["ideal_ms"] = round(ideal_ms, 4)
    roof["fp32_only_frac"] = round(roof["achieved"] / FP32_MFMA_PEAK_TFLOPS, 4)
    hnet_ms = sum(per_op[n] for n in ("route+compact stage1", "route+compact stage2", "dechunk stage2", "dechunk stage1"))
    hnet_bytes = sum(alg[n]["bytes"] for n in ("route+compact stage1", "route+compact stage2", "dechunk stage2", "dechunk stage1"))
    # each layer also timed as the chain it runs as (its ops queued back to
    # back on one stream, the Infinity Cache flushed once before)
    chains = time_ops(wl, ops=[("hnet", lambda: [f() for _, f in wl.hnet_ops()]),
                               ("byteflow", lambda: [f() for _, f in wl.byteflow_ops()])])
    out = {
        "metric": "chunked bytes/sec at T=8192 (route+compact+dechunk, ΔR+TopK); % roofline",
        "value": wl.N / (ms * 1e-3),
        "unit": "bytes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "hnet_2stage_T8192_B32 + byteflow_T8192_B32_K2048", "global_batch": 32,
                   "seq_len": 8192, "hnet": {"d_local": 512, "d_mid": 768, "stage_quantile": 0.75,
                                             "M1": wl.M1, "M2": wl.M2},
                   "byteflow": {"d_local": 512, "d_global": 1536, "K": 2048, "bins": 16, "eps2": 0.5,
                                "upsample_items": wl.up_items},
                   "parallelism": "single GPU",
                   "schedule": SCHEDULES[args.schedule]},
        "roofline": roof,
        "step_roofline": step_roofline(alg, ms),
        "other_schedules": {sch: {"schedule": SCHEDULES[sch], "ms_per_step": round(t[0], 4),
                                  "value": wl.N / (t[0] * 1e-3), "coding_rate_ms": round(t[1], 4)}
                            for sch, t in others.items()},
        "dominant_op": dom_name,
        "breakdown": breakdown,
        "hnet_layer": {"ms": round(hnet_ms, 4), "bytes_per_s": wl.N / (hnet_ms * 1e-3),
                       "hbm_GBps": round(hnet_bytes / (hnet_ms * 1e-3) / 1e9, 1),
                       "hbm_frac": round(hnet_bytes / (hnet_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "basis": "sum of the four ops' medians, each timed alone from a flushed cache",
                       "chained_ms": round(chains["hnet"], 4),
                       "chained_hbm_frac": round(hnet_bytes / (chains["hnet"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "byteflow_layer": {"chained_ms": round(chains["byteflow"], 4),
                           "basis": "coding rate, Top-K, gather and upsample queued back to back from a flushed "
                                    "cache"},
    }
    nxt = {}
    nalg = wl.next_algorithmic()
    for name, t in time_ops(wl, ops=wl.next_ops()).items():
        nxt[name] = op_rates(nalg[name], t)
    out["next_rows"] = nxt
    out["status_word"] = int(wl.st.item())  # 0: no capacity overflow, non-finite value or abandoned wait
    log("timing the other workloads")
    out["other_workloads"] = other_workloads(wl.B, torch)
    if not args.no_cpu_baseline:
        log("timing the oracle baseline on the host")
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
