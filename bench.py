#!/usr/bin/env python3
"""Benchmark of blockwise absmax quantization / dequantization on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
  1. bq_quantize_nested    bf16, n = 2^29 (1 GiB), 4-bit codes, B = 64, nested statistics
                           (256-entry table, groups of 256 blocks)
  2. bq_dequantize_nested  the same tensor back to bf16
  3. bq_dequant_q32        4096 x 14336 GGUF-style 4-bit blocks (18 B) to bf16
  4. bq_dequant_q32        4096 x 14336 GGUF-style 8-bit blocks (34 B) to bf16
Inputs are generated on the device before timing (they are resident in HBM when the timed
region starts).  `value` is input bytes of the step / step time (the metric's "effective
GB/s (input bytes)"); every call's algorithmic read+write bytes against the 8 TB/s HBM peak
is in `detail`.  `roofline` is the slower of the two 1 GiB kernels as the step launches them,
the data kernel of bq_quantize_nested and the one kernel of bq_dequantize_nested, each timed
with HIP events on the stream it runs on over further steps right after the timed region, as
the difference of two event spans that share a marker's lead (see kernel_step_loop).  `cpu_baseline` is
the CPU oracle on the whole step input from as many host threads as the oracle may use (at
most 16), plus the same oracle on one thread over a sixteenth of the step; the threaded
oracle's outputs are also this run's parity reference (`parity`: every output byte of the
step's calls against the oracle's).

    python bench.py [--gpus 1] [--steps 20] [--warmup 40] [--no-detail] [--no-cpu-baseline]
    python bench.py --profile     (a few launches of each kernel, the bf16 2^26 8-bit calls, the
                                   IQ2_XS and IQ1_S encode / decode and the fused GEMM at
                                   14336 x 4096, then a 1 GiB copy, for rocprofv3)
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective GB/s (input bytes) and % of HBM peak, quantize + dequantize"
PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
KERNEL_SOURCES = {
    "quantize_kernel": "dequantization_block_absmax_amd/csrc/k_quant.hip",
    "dequantize_nested_kernel": "dequantization_block_absmax_amd/csrc/k_dequant.hip",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # 40 warm-up steps (about 22 ms): the first ~15 ms of back-to-back steps run 3-5% slower
    # while the GPU's clocks settle; the timed steps measure the sustained rate after that.
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--no-detail", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--profile", action="store_true")
    return p.parse_args()


class Workload:
    """The 1 GiB bf16 nested 4-bit workload and the GGUF 4096 x 14336 blocks, resident on the device."""

    N5, B5, B2 = 1 << 29, 64, 256
    ROWS, COLS = 4096, 14336

    def __init__(self, bq, synth, torch, dev):
        self.bq, self.torch = bq, torch
        # code tables converted to the C struct once (not on every call)
        self.t16, self.t256 = bq.code_table(synth.table16()), bq.code_table(synth.table256())
        self.t16_np, self.t256_np = synth.table16(), synth.table256()
        n, B, B2 = self.N5, self.B5, self.B2
        self.nb = bq.num_blocks(n, B)
        self.ng = bq.num_blocks(self.nb, B2)
        self.x = synth.blockwise_input(n, "bfloat16", 5, std=0.02, device=dev)
        self.packed = torch.empty(n // 2, dtype=torch.uint8, device=dev)
        self.ws_bytes = bq.bq_nested_workspace_bytes(n, B, B2)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.q2 = torch.empty(self.nb, dtype=torch.uint8, device=dev)
        self.absmax2 = torch.empty(self.ng, dtype=torch.float32, device=dev)
        self.mean = torch.empty(1, dtype=torch.float32, device=dev)
        self.out = torch.empty(n, dtype=torch.bfloat16, device=dev)
        self.stats = bq.nested_stats(self.q2, self.absmax2, self.mean, self.t256, B2, self.ws, self.ws_bytes)
        self.absmax = self.ws[: self.nb * 4].view(torch.float32)
        self.n4 = self.ROWS * self.COLS
        self.q4 = synth.q32_blocks(self.n4 // 32, "q4", seed=4, device=dev)
        self.q8 = synth.q32_blocks(self.n4 // 32, "q8", seed=4, device=dev)
        self.out4 = torch.empty(self.n4, dtype=torch.bfloat16, device=dev)
        self.out8 = torch.empty(self.n4, dtype=torch.bfloat16, device=dev)
        self.q32_sets = {}  # rotated GGUF buffer sets of the per-call timing
        e = 2 ** 29
        # input bytes and algorithmic read+write bytes of each call
        self.calls = {
            "quantize_nested": dict(inp=2 * e, rw=2 * e + e // 2 + self.nb + 4 * self.ng + 4),
            "dequantize_nested": dict(inp=e // 2 + self.nb + 4 * self.ng + 4, rw=2 * e + e // 2 + self.nb + 4 * self.ng + 4),
            "dequant_q32_q4": dict(inp=self.n4 // 32 * 18, rw=self.n4 // 32 * 18 + 2 * self.n4),
            "dequant_q32_q8": dict(inp=self.n4 // 32 * 34, rw=self.n4 // 32 * 34 + 2 * self.n4),
        }

    def time_q32_rotated(self, name, time_calls, reps):
        """Mean ms of a GGUF call over buffer sets rotated to defeat the last-level cache."""
        bq, torch = self.bq, self.torch
        src = self.q4 if name == "dequant_q32_q4" else self.q8
        fmt = bq.BQ_Q32_Q4 if name == "dequant_q32_q4" else bq.BQ_Q32_Q8
        if name not in self.q32_sets:  # made once, kept for the later rounds
            k = -(-(1 << 30) // (src.numel() + 2 * self.n4))
            self.q32_sets[name] = [(src.clone(), torch.empty_like(self.out4)) for _ in range(k)]
        sets = self.q32_sets[name]
        i = [0]

        def call():
            blocks, out = sets[i[0] % len(sets)]
            i[0] += 1
            bq.check(bq.bq_dequant_q32(blocks, bq.BQ_BF16, self.n4, self.COLS, fmt, out), name)
        return time_calls(call, torch, reps)

    def run(self, name):
        bq = self.bq
        if name == "quantize_nested":
            st = bq.bq_quantize_nested(self.x, bq.BQ_BF16, self.N5, self.B5, self.t16, self.stats, self.packed)
        elif name == "dequantize_nested":
            st = bq.bq_dequantize_nested(self.out, bq.BQ_BF16, self.N5, self.B5, self.t16, self.stats, self.packed)
        elif name == "dequant_q32_q4":
            st = bq.bq_dequant_q32(self.q4, bq.BQ_BF16, self.n4, self.COLS, bq.BQ_Q32_Q4, self.out4)
        elif name == "dequant_q32_q8":
            st = bq.bq_dequant_q32(self.q8, bq.BQ_BF16, self.n4, self.COLS, bq.BQ_Q32_Q8, self.out8)
        elif name == "quantize_kernel":  # the data kernel of quantize_nested on its own
            st = bq.bq_quantize_blockwise(self.x, bq.BQ_BF16, self.N5, self.B5, self.t16, self.absmax, self.packed)
        else:
            raise KeyError(name)
        bq.check(st, name)


class TimingEvents:
    """HIP events created with hipEventDisableSystemFence, through the HIP runtime torch has
    loaded (dlopen of the same path returns the same library), for the kernel launches that
    stamp their own start and end (hipExtLaunchKernel, armed by bq_debug_time_next_kernel).
    Events recorded between kernels instead put a marker packet there, which on MI355X left
    about 5 us of idle GPU on each side of the bracketed kernel and counted it in the kernel's
    time.  Read them after a device synchronization."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, torch):
        import ctypes
        import re
        self.torch = torch
        torch.cuda.init()
        with open("/proc/self/maps") as f:
            paths = sorted(set(re.findall(r"(/\S*libamdhip64\S*)", f.read())))
        if not paths:
            raise RuntimeError("the HIP runtime torch uses is not loaded")
        self.hip = ctypes.CDLL(paths[0])
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.c_void_p, ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ctypes = ctypes
        self.made = []

    def new(self) -> int:
        ev = self.ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ctypes.byref(ev), self.FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.made.append(ev.value)
        return ev.value

    def record(self, ev: int, stream: int):
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a: int, b: int) -> float:
        out = self.ctypes.c_float()
        if self.hip.hipEventElapsedTime(self.ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for ev in self.made:
            self.hip.hipEventDestroy(ev)
        self.made = []


STEP = ["quantize_nested", "dequantize_nested", "dequant_q32_q4", "dequant_q32_q8"]
ROUNDS, REPS = 7, 10  # per-call breakdown: interleaved rounds of back-to-back calls


def timed_step_loop(w: Workload, torch, steps: int):
    """Runs `steps` steps between two HIP events on the current stream (the stream every call
    is enqueued on), with nothing between the kernels; returns the elapsed ms of the whole
    region and the host wall ms."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        for name in STEP:
            w.run(name)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b), (time.perf_counter() - t0) * 1e3


def kernel_step_loop(w: Workload, bq, torch, cycles: int, tev: TimingEvents):
    """Steps again, right after the timed region, in cycles of four, timing the in-step
    launches of the nested-quantize data kernel Q and of the nested-dequantize kernel D with
    HIP events on the stream they run on.  A marker recorded before a launch leads it by a
    near-constant few microseconds of idle GPU (a marker's latency), and a stop event bound to
    a launch (bq_debug_time_next_kernel) takes the kernel's end, then idles the GPU for a few
    microseconds after it.  So each kernel's time is the difference of two spans that open
    with the same kind of marker:
      step 2: marker before the previous step's Q8 dequant, stop bound to Q   (lead + Q8 + Q)
      step 3: marker before Q8, stop bound to Q8                              (lead + Q8)
      step 2: marker before D, stop bound to the Q4 dequant after it          (lead + D + Q4)
      step 3: marker before Q4, stop bound to Q4                              (lead + Q4)
    Inside a span nothing idles: Q runs right after Q8 and Q4 right after D, as in the timed
    steps.  Returns (Q spans, Q8 spans, D spans, Q4 spans) in ms."""
    spans = {k: [] for k in ("q", "q8", "d", "q4")}
    arm = bq.bq_debug_time_next_kernel
    stream = torch.cuda.current_stream().cuda_stream

    def marker():
        ev = tev.new()
        tev.record(ev, stream)
        return ev

    def stop_on(name):
        ev = tev.new()
        bq.check(arm(None, ev), "arm")
        w.run(name)
        return ev

    torch.cuda.synchronize()
    for _ in range(cycles):
        w.run("quantize_nested")                       # step 1
        w.run("dequantize_nested")
        w.run("dequant_q32_q4")
        m = marker()
        w.run("dequant_q32_q8")
        spans["q"].append((m, stop_on("quantize_nested")))  # step 2
        m = marker()
        w.run("dequantize_nested")
        spans["d"].append((m, stop_on("dequant_q32_q4")))
        w.run("dequant_q32_q8")
        w.run("quantize_nested")                       # step 3
        w.run("dequantize_nested")
        m = marker()
        spans["q4"].append((m, stop_on("dequant_q32_q4")))
        m = marker()
        spans["q8"].append((m, stop_on("dequant_q32_q8")))
        for name in STEP:                              # step 4
            w.run(name)
    torch.cuda.synchronize()
    return tuple([tev.ms(x, y) for x, y in spans[k]] for k in ("q", "q8", "d", "q4"))


def time_calls(fn, torch, reps: int) -> float:
    """Mean ms of fn() over reps back-to-back calls, HIP events on the current stream."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def source_digest(path: str) -> str:
    h = hashlib.sha256()
    for p in sorted([os.path.join(ROOT, path), os.path.join(ROOT, "dequantization_block_absmax_amd/csrc/bq_device.h"),
                     os.path.join(ROOT, "dequantization_block_absmax_amd/csrc/bq_internal.h")]):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_for(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % kernel)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return t.get("hbm_bytes_per_launch")


def detail_configs(bq, synth, torch, dev, peak):
    """fp32 2^19, fp16 2^23 + 1 (every block size) and bf16 2^26 8-bit calls on their own, with
    buffer sets rotated so that each call's data is not resident in the 256 MB last-level cache."""
    out = {}
    t16, t256 = bq.code_table(synth.table16()), bq.code_table(synth.table256())

    def rotate(make, footprint, fn, reps, graph=False):
        """Ms per call over buffer sets rotated past the last-level cache (the median of
        ROUNDS batches of reps back-to-back calls); with graph, also the ms per call when the k
        calls are captured once as a HIP graph and replayed (no per-call launch cost from the
        host)."""
        k = max(1, min(64, -(-(1 << 30) // footprint)))
        sets = [make() for _ in range(k)]
        i = [0]

        def call():
            fn(sets[i[0] % k])
            i[0] += 1
        ms = statistics.median(time_calls(call, torch, reps) for _ in range(ROUNDS))
        if not graph:
            return ms, None
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for st in sets:
                fn(st)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for st in sets:
                fn(st)
        replays = max(1, reps // k)
        gms = statistics.median(time_calls(g.replay, torch, replays) for _ in range(ROUNDS)) / k
        del g
        return ms, gms

    def rec(name, ms, inp, rw, graph_ms=None):
        out[name] = dict(us=round(ms * 1e3, 2), input_gbs=round(inp / ms / 1e6, 1), rw_gbs=round(rw / ms / 1e6, 1),
                         pct_hbm_peak=round(100 * rw / ms / 1e6 / peak, 1))
        if graph_ms is not None:  # the same calls replayed from a HIP graph
            out[name].update(us_graph=round(graph_ms * 1e3, 2),
                             pct_hbm_peak_graph=round(100 * rw / graph_ms / 1e6 / peak, 1))

    def blockwise(tag, n, dtype, B, table, seed, std, p_out=0.0, p_nf=0.0, reps=50):
        es = {"float32": 4, "float16": 2, "bfloat16": 2}[dtype]
        tdt = {"float32": torch.float32, "float16": torch.float16, "bfloat16": torch.bfloat16}[dtype]
        code = {"float32": bq.BQ_F32, "float16": bq.BQ_F16, "bfloat16": bq.BQ_BF16}[dtype]
        x0 = synth.blockwise_input(n, dtype, seed, std=std, p_out=p_out, p_nf=p_nf, device=dev)
        K = table.size
        nb = bq.num_blocks(n, B)
        pb = bq.packed_bytes(n, K)

        def make():
            return dict(x=x0.clone(), a=torch.empty(nb, dtype=torch.float32, device=dev),
                        p=torch.empty(pb + 16, dtype=torch.uint8, device=dev), o=torch.empty(n, dtype=tdt, device=dev))
        foot = n * es * 2 + pb + nb * 4
        small = n * es < (64 << 20)  # launch-bound sizes: also time them replayed from a graph
        qms, qg = rotate(make, foot, lambda s: bq.check(bq.bq_quantize_blockwise(s["x"], code, n, B, table, s["a"],
                                                                                 s["p"])), reps, small)
        sets_once = make()
        bq.check(bq.bq_quantize_blockwise(sets_once["x"], code, n, B, table, sets_once["a"], sets_once["p"]))
        dms, dg = rotate(lambda: dict(a=sets_once["a"].clone(), p=sets_once["p"].clone(),
                                      o=torch.empty(n, dtype=tdt, device=dev)),
                         foot, lambda s: bq.check(bq.bq_dequantize_blockwise(s["o"], code, n, B, table, s["a"],
                                                                             s["p"])), reps, small)
        rw = n * es + pb + nb * 4
        rec(tag + " quantize", qms, n * es, rw, qg)
        rec(tag + " dequantize", dms, pb + nb * 4, rw, dg)

    blockwise("fp32 n=2^19 4-bit B=64", 524288, "float32", 64, t16, 1, 1.0, reps=200)
    for B in (32, 64, 128, 256, 512, 1024, 2048, 4096):
        blockwise("fp16 n=2^23+1 4-bit B=%d" % B, 8388609, "float16", B, t16, 2, 1.0, 1e-3, 1e-4, reps=100)
    blockwise("bf16 n=2^26 8-bit B=4096", 1 << 26, "bfloat16", 4096, t256, 3, 0.02, reps=50)
    out.update(loading_pipeline(bq, synth, torch, dev, t16))
    out.update(fused_linear(bq, synth, torch, dev, t16, t256, peak))
    out.update(iq2xs(bq, synth, torch, dev))
    return out


def fused_linear(bq, synth, torch, dev, t16, t256, peak, N=14336, K=4096, B=64, sets=24):
    """bq_linear_blockwise at a decode shape (a 14336 x 4096 weight, bf16 activations) for M = 1
    and 4, and bq_gemm_blockwise for M = 16, 64, 256, 512 and 1024, 4- and 8-bit codes, with the weights
    rotated over enough sets to miss the 256 MB last-level cache.  Beside each, the unfused
    path: dequantize to bf16 with this library, then torch's matmul."""
    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    for KB, table in ((4, t16), (8, t256)):
        per = N * K // 2 if KB == 4 else N * K
        ws = [(torch.randint(0, 256, (per,), dtype=torch.uint8, device=dev, generator=g),
               (0.02 * torch.exp(torch.randn(N * K // B, device=dev, generator=g))).float()) for _ in range(sets)]
        wbf = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
        for M in (1, 4):
            x = torch.randn(M, K, device=dev, generator=g).to(torch.bfloat16)
            y = torch.empty(M, N, device=dev)
            i = [0]

            def fused():
                p, a = ws[i[0] % sets]
                i[0] += 1
                bq.check(bq.bq_linear_blockwise(x, bq.BQ_BF16, M, K, N, B, table, a, p, y))

            def unfused():
                p, a = ws[i[0] % sets]
                i[0] += 1
                bq.check(bq.bq_dequantize_blockwise(wbf, bq.BQ_BF16, N * K, B, table, a, p))
                torch.matmul(x, wbf.t())
            fused()
            unfused()
            torch.cuda.synchronize()
            f_ms = statistics.median(time_calls(fused, torch, 48) for _ in range(ROUNDS))
            u_ms = statistics.median(time_calls(unfused, torch, 24) for _ in range(ROUNDS))
            # the same calls captured once as a HIP graph and replayed: a call this short is
            # otherwise bound by the host's launch rate
            gr = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(sets):
                    fused()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(gr):
                for _ in range(sets):
                    fused()
            g_ms = statistics.median(time_calls(gr.replay, torch, 2) for _ in range(ROUNDS)) / sets
            del gr
            byts = per + 4 * (N * K // B) + 2 * M * K + 4 * M * N
            out["linear %dx%d %d-bit B=%d M=%d bf16" % (N, K, KB, B, M)] = dict(
                us=round(f_ms * 1e3, 2), rw_gbs=round(byts / f_ms / 1e6, 1),
                pct_hbm_peak=round(100 * byts / f_ms / 1e6 / peak, 1),
                us_graph=round(g_ms * 1e3, 2), pct_hbm_peak_graph=round(100 * byts / g_ms / 1e6 / peak, 1),
                unfused_us=round(u_ms * 1e3, 2), speedup_vs_unfused=round(u_ms / f_ms, 2))
        for M in (16, 64, 256, 512, 1024):  # bq_gemm_blockwise: 16-bit weights on the matrix cores
            x = torch.randn(M, K, device=dev, generator=g).to(torch.bfloat16)
            y = torch.empty(M, N, device=dev)
            i = [0]

            def fused():
                p, a = ws[i[0] % sets]
                i[0] += 1
                bq.check(bq.bq_gemm_blockwise(x, bq.BQ_BF16, M, K, N, B, table, a, p, y))

            def unfused():
                p, a = ws[i[0] % sets]
                i[0] += 1
                bq.check(bq.bq_dequantize_blockwise(wbf, bq.BQ_BF16, N * K, B, table, a, p))
                torch.matmul(x, wbf.t())
            fused()
            unfused()
            torch.cuda.synchronize()
            f_ms = statistics.median(time_calls(fused, torch, 24) for _ in range(ROUNDS))
            u_ms = statistics.median(time_calls(unfused, torch, 24) for _ in range(ROUNDS))
            byts = per + 4 * (N * K // B) + 2 * M * K + 4 * M * N
            out["gemm %dx%d %d-bit B=%d M=%d bf16" % (N, K, KB, B, M)] = dict(
                us=round(f_ms * 1e3, 2), tflops=round(2 * M * N * K / f_ms / 1e9, 1),
                pct_bf16_mfma_peak=round(100 * 2 * M * N * K / f_ms / 1e9 / 2500.0, 1),
                pct_hbm_peak=round(100 * byts / f_ms / 1e6 / peak, 1),
                unfused_us=round(u_ms * 1e3, 2), speedup_vs_unfused=round(u_ms / f_ms, 2))
        del ws, wbf
    return out


FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector peak (FMA = 2 flops, dual-issue / packed)


def iq2xs(bq, synth, torch, dev, rows=4096, cols=14336, sets=4):
    """The IQ2_XS- and IQ1_S-style encoders and decoders on a 4096 x 14336 bf16 weight (229,376
    superblocks).  The encoder is a search bound by VALU issue: its algorithmic work per
    superblock is 32 vectors x 512 entries x (an 8-term dot, 8 FMA, plus 2 FMA of the error
    for each of the 16 local scales), 1,310,720 flops counting an FMA as two, reported against
    the fp32 vector peak.  The decoder is bound by HBM (74 bytes in, 512 out per superblock)."""
    n = rows * cols
    nb = n // 256
    x = synth.blockwise_input(n, "bfloat16", 40, std=0.02, p_out=0.01, device=dev)
    scales = synth.iq2xs_scales(x)
    grid = torch.from_numpy(synth.iq2xs_grid().reshape(-1)).to(dev)
    blocks = torch.empty(nb * 74, dtype=torch.uint8, device=dev)
    rejected = torch.zeros(1, dtype=torch.int32, device=dev)
    outs = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(sets)]

    def enc():
        bq.check(bq.bq_iq2xs_quantize(x, bq.BQ_BF16, n, cols, grid, scales, blocks, rejected), "iq2xs quantize")
    i = [0]

    def dec():
        out = outs[i[0] % sets]
        i[0] += 1
        bq.check(bq.bq_iq2xs_dequantize(blocks, grid, n, cols, bq.BQ_BF16, out), "iq2xs dequantize")
    enc()
    e_ms = statistics.median(time_calls(enc, torch, 3) for _ in range(ROUNDS))
    d_ms = statistics.median(time_calls(dec, torch, 8) for _ in range(ROUNDS))
    flops = nb * 32 * 512 * (16 + 16 * 4)
    dec_bytes = nb * 74 + 2 * n
    out = {"iq2xs encode bf16 4096x14336 (search over a 512-entry grid)": dict(
               us=round(e_ms * 1e3, 1), superblocks_per_s=round(nb / e_ms * 1e3, 1),
               tflops=round(flops / e_ms / 1e9, 1),
               pct_fp32_vector_peak=round(100 * flops / e_ms / 1e9 / FP32_VECTOR_PEAK_TFLOPS, 1)),
           "iq2xs decode to bf16 4096x14336": dict(
               us=round(d_ms * 1e3, 2), rw_gbs=round(dec_bytes / d_ms / 1e6, 1),
               pct_hbm_peak=round(100 * dec_bytes / d_ms / 1e6 / PEAK_GBS, 1))}
    # IQ1_S-style: 32 vectors x 2048 entries x (an 8-term dot, 8 FMA; two shifted dots, 2 FMA;
    # 2 FMA of the error for each of the 16 choices) per superblock, FMA = 2 flops.
    grid1 = torch.from_numpy(synth.iq1s_grid().reshape(-1)).to(dev)
    blocks1 = torch.empty(nb * 50, dtype=torch.uint8, device=dev)

    def enc1():
        bq.check(bq.bq_iq1s_quantize(x, bq.BQ_BF16, n, cols, grid1, blocks1), "iq1s quantize")
    i[0] = 0

    def dec1():
        o = outs[i[0] % sets]
        i[0] += 1
        bq.check(bq.bq_iq1s_dequantize(blocks1, grid1, n, cols, bq.BQ_BF16, o), "iq1s dequantize")
    enc1()
    e1_ms = statistics.median(time_calls(enc1, torch, 2) for _ in range(ROUNDS))
    d1_ms = statistics.median(time_calls(dec1, torch, 8) for _ in range(ROUNDS))
    flops1 = nb * 32 * 2048 * (16 + 4 + 16 * 4)
    dec1_bytes = nb * 50 + 2 * n
    out["iq1s encode bf16 4096x14336 (search over a 2048-entry grid)"] = dict(
        us=round(e1_ms * 1e3, 1), superblocks_per_s=round(nb / e1_ms * 1e3, 1), tflops=round(flops1 / e1_ms / 1e9, 1),
        pct_fp32_vector_peak=round(100 * flops1 / e1_ms / 1e9 / FP32_VECTOR_PEAK_TFLOPS, 1))
    out["iq1s decode to bf16 4096x14336"] = dict(
        us=round(d1_ms * 1e3, 2), rw_gbs=round(dec1_bytes / d1_ms / 1e6, 1),
        pct_hbm_peak=round(100 * dec1_bytes / d1_ms / 1e6 / PEAK_GBS, 1))
    return out


def loading_pipeline(bq, synth, torch, dev, table, chunks=8, chunk=1 << 25, B=64):
    """The loading path: bf16 weights in pinned host memory reach the device in chunks on one
    stream while a second stream quantizes each chunk as it lands (double-buffered).  Reports
    the rate of the whole pipeline next to the host-to-device copies alone: the library's
    calls take device pointers, so PCIe is outside the boundary and never part of `value`."""
    x = synth.blockwise_input(chunks * chunk, "bfloat16", 8, std=0.02, device=dev)
    host = torch.empty(chunks * chunk, dtype=torch.bfloat16, pin_memory=True)
    host.copy_(x)
    del x
    bufs = [torch.empty(chunk, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    nb = chunk // B
    absmax = torch.empty(chunks, nb, dtype=torch.float32, device=dev)
    packed = torch.empty(chunks, chunk // 2, dtype=torch.uint8, device=dev)
    copy_s, work_s = torch.cuda.Stream(), torch.cuda.Stream()

    def run(quantize):
        copied = [torch.cuda.Event() for _ in range(chunks)]
        used = [torch.cuda.Event() for _ in range(chunks)]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(copy_s)
        for c in range(chunks):
            buf = bufs[c % 2]
            if c >= 2:
                copy_s.wait_event(used[c - 2])
            with torch.cuda.stream(copy_s):
                buf.copy_(host[c * chunk:(c + 1) * chunk], non_blocking=True)
                copied[c].record(copy_s)
            work_s.wait_event(copied[c])
            if quantize:
                bq.check(bq.bq_quantize_blockwise(buf, bq.BQ_BF16, chunk, B, table, absmax[c], packed[c], work_s))
            used[c].record(work_s)
        copy_s.wait_event(used[chunks - 1])
        b.record(copy_s)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    run(True)
    copy_ms = statistics.median(run(False) for _ in range(3))
    pipe_ms = statistics.median(run(True) for _ in range(3))
    byts = chunks * chunk * 2
    return {"loading pipeline bf16 2^28 in 8 chunks: pinned H2D + 4-bit B=64 quantize": dict(
        us=round(pipe_ms * 1e3, 1), input_gbs=round(byts / pipe_ms / 1e6, 1),
        h2d_only_us=round(copy_ms * 1e3, 1), h2d_only_gbs=round(byts / copy_ms / 1e6, 1),
        quantize_hidden=round(copy_ms / pipe_ms, 3))}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def step_outputs(w: Workload, torch):
    """Host copies of every output of one step (the last one run)."""
    import numpy as np

    def bits(t):
        return t.cpu().view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.cpu().numpy()
    return dict(packed=w.packed.cpu().numpy(), q2=w.q2.cpu().numpy(), absmax2=w.absmax2.cpu().numpy(),
                mean=w.mean.cpu().numpy()[:1], out=bits(w.out), out4=bits(w.out4), out8=bits(w.out8))


def oracle_step(o, w: Workload, xs, b4, b8, n5: int, rows: int) -> dict:
    """The oracle on the first n5 elements of the 1 GiB tensor and the first `rows` rows of
    both GGUF matrices: the calls of one step, in order."""
    import numpy as np

    import oracle
    r = o.quantize_nested(xs[:n5], oracle.BF16, w.B5, w.t16_np, w.t256_np, w.B2)
    out = o.dequantize_nested(r["packed"], r["q2"], r["absmax2"], r["mean"], n5, oracle.BF16, w.B5, w.t16_np,
                              w.t256_np, w.B2)
    m = rows * w.COLS
    out4 = o.dequant_q32(b4[:m // 32 * 18], m, w.COLS, oracle.Q4, oracle.BF16)
    out8 = o.dequant_q32(b8[:m // 32 * 34], m, w.COLS, oracle.Q8, oracle.BF16)
    return dict(packed=r["packed"], q2=r["q2"], absmax2=r["absmax2"], mean=np.float32([r["mean"]]), out=out,
                out4=out4, out8=out8)


def step_input_bytes(w: Workload, n5: int, rows: int) -> int:
    nb = n5 // w.B5
    q2_in = n5 // 2 + nb + 4 * (-(-nb // w.B2)) + 4
    return 2 * n5 + q2_in + rows * w.COLS // 32 * (18 + 34)


def cpu_baseline_and_parity(w: Workload, torch, gpu: dict):
    """The CPU oracle as it stands, on this run's inputs.  (i) The whole step from as many host
    threads as the oracle uses (contiguous ranges of whole blocks, groups and rows; at most
    16); its outputs are compared byte for byte with the step's GPU outputs.  (ii) One thread
    over a sixteenth of the step (the first 2^25 elements and 256 rows), the single-core rate."""
    import numpy as np

    import oracle
    xs = w.x.cpu().view(torch.int16).numpy().view(np.uint16)
    b4, b8 = w.q4.cpu().numpy(), w.q8.cpu().numpy()
    po = oracle.ParallelOracle()
    t0 = time.perf_counter()
    ref = oracle_step(po, w, xs, b4, b8, w.N5, w.ROWS)
    dt_n = time.perf_counter() - t0
    mismatched = []
    for k, v in ref.items():
        g = gpu[k][:v.size]
        if g.shape != v.shape or not np.array_equal(g.view(np.uint8), np.ascontiguousarray(v).view(np.uint8)):
            mismatched.append(k)
    del ref
    o1 = oracle.Oracle()
    n1, rows1 = w.N5 // 16, w.ROWS // 16
    t0 = time.perf_counter()
    oracle_step(o1, w, xs, b4, b8, n1, rows1)
    dt_1 = time.perf_counter() - t0
    full = step_input_bytes(w, w.N5, w.ROWS)
    part = step_input_bytes(w, n1, rows1)
    cpu = dict(value=round(full / dt_n / 1e9, 4), unit="GB/s", cores=po.threads, kind="oracle",
               sample="the whole step input (bf16 2^29 nested quantize + dequantize, both 4096x14336 GGUF "
                      "matrices) on %d host threads over contiguous ranges of whole blocks, groups and rows: "
                      "%.1f s" % (po.threads, dt_n),
               cpu_model=cpu_model(), os_cpu_count=os.cpu_count(),
               single_thread=dict(value=round(part / dt_1 / 1e9, 4), unit="GB/s", cores=1,
                                  sample="first 2^25 elements and first 256 rows (1/16 of the step): %.1f s" % dt_1))
    parity = dict(ok=not mismatched, mismatched=mismatched,
                  compared="every byte of packed, q2, absmax2, mean, the nested dequantize and both GGUF outputs "
                           "of the last timed step against the threaded oracle")
    return cpu, parity


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: each GPU would run these kernels on its own shard of "
              "whole blocks, with no communication except, for nested statistics, one all-gather of "
              "8-byte partial sums of the mean; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import dequantization_block_absmax_amd as bq
    import synth

    dev = torch.device("cuda:0")
    log("generating inputs on", torch.cuda.get_device_name(0))
    w = Workload(bq, synth, torch, dev)
    torch.cuda.synchronize()

    if args.profile:
        for name in STEP + ["quantize_kernel"]:
            for _ in range(3):
                w.run(name)
        # the bf16 2^26 8-bit B=4096 workload's two calls, for their own counter summaries
        n3 = 1 << 26
        x3 = synth.blockwise_input(n3, "bfloat16", 3, std=0.02, device=dev)
        a3 = torch.empty(n3 // 4096, dtype=torch.float32, device=dev)
        p3 = torch.empty(n3, dtype=torch.uint8, device=dev)
        o3 = torch.empty_like(x3)
        for _ in range(3):
            bq.check(bq.bq_quantize_blockwise(x3, bq.BQ_BF16, n3, 4096, w.t256, a3, p3), "bf16 2^26 8-bit quantize")
        for _ in range(3):
            bq.check(bq.bq_dequantize_blockwise(o3, bq.BQ_BF16, n3, 4096, w.t256, a3, p3), "bf16 2^26 8-bit dequantize")
        # the IQ2_XS-style encoder and decoder on a 4096 x 14336 bf16 weight
        n6, cols6 = 4096 * 14336, 14336
        x6 = synth.blockwise_input(n6, "bfloat16", 40, std=0.02, p_out=0.01, device=dev)
        s6 = synth.iq2xs_scales(x6)
        g6 = torch.from_numpy(synth.iq2xs_grid().reshape(-1)).to(dev)
        b6 = torch.empty(n6 // 256 * 74, dtype=torch.uint8, device=dev)
        r6 = torch.zeros(1, dtype=torch.int32, device=dev)
        o6 = torch.empty(n6, dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            bq.check(bq.bq_iq2xs_quantize(x6, bq.BQ_BF16, n6, cols6, g6, s6, b6, r6), "iq2xs quantize")
        for _ in range(3):
            bq.check(bq.bq_iq2xs_dequantize(b6, g6, n6, cols6, bq.BQ_BF16, o6), "iq2xs dequantize")
        g7 = torch.from_numpy(synth.iq1s_grid().reshape(-1)).to(dev)
        b7 = torch.empty(n6 // 256 * 50, dtype=torch.uint8, device=dev)
        for _ in range(3):
            bq.check(bq.bq_iq1s_quantize(x6, bq.BQ_BF16, n6, cols6, g7, b7), "iq1s quantize")
        for _ in range(3):
            bq.check(bq.bq_iq1s_dequantize(b7, g7, n6, cols6, bq.BQ_BF16, o6), "iq1s dequantize")
        del x6, o6
        # the fused dequantize + GEMM on a 14336 x 4096 weight at M = 256, 512 and 1024 (the
        # 128 x 128, 256 x 128 and 256 x 256 tile forms), 4- and 8-bit codes
        gN, gK = 14336, 4096
        gen = torch.Generator(device=dev)
        gen.manual_seed(5)
        for table, per in ((w.t16, gN * gK // 2), (w.t256, gN * gK)):
            gp = torch.randint(0, 256, (per,), dtype=torch.uint8, device=dev, generator=gen)
            ga = (0.02 * torch.exp(torch.randn(gN * gK // 64, device=dev, generator=gen))).float()
            for M in (256, 512, 1024):
                gx = torch.randn(M, gK, device=dev, generator=gen).to(torch.bfloat16)
                gy = torch.empty(M, gN, device=dev)
                for _ in range(3):
                    bq.check(bq.bq_gemm_blockwise(gx, bq.BQ_BF16, M, gK, gN, 64, table, ga, gp, gy), "gemm")
            del gp, ga, gx, gy
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)  # a plain 1 GiB copy for counter calibration
        torch.cuda.synchronize()
        log("profile pass done")
        return

    # No garbage collection inside timed regions: a collection pass over the process's objects
    # stalls the host for milliseconds and shows up as idle GPU time between launches.
    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        for name in STEP:
            w.run(name)
    total_ms, wall_ms = timed_step_loop(w, torch, args.steps)
    ms_per_step = total_ms / args.steps
    gpu_out = None if args.no_cpu_baseline else step_outputs(w, torch)  # the last timed step's outputs
    tev = TimingEvents(torch)
    q_sp, q8_sp, d_sp, q4_sp = kernel_step_loop(w, bq, torch, args.steps, tev)
    tev.close()
    # Per-call breakdown: each call back to back between two events (an event between calls
    # adds a few microseconds of its own), REPS calls per round.  The GGUF calls rotate over
    # buffer sets of more than 1 GiB in total, so that back-to-back calls do not find their data
    # in the 256 MB last-level cache (inside the step, the 1 GiB calls between them evict it
    # anyway).
    # The call types take turns over several rounds and each reports its median round: clocks
    # drift under sustained load, and a fixed order would hand the drift to whichever call is
    # timed at the wrong moment.
    rounds = {name: [] for name in STEP + ["quantize_kernel"]}  # + the blockwise quantize alone
    for _ in range(ROUNDS):
        for name in rounds:
            if name.startswith("dequant_q32"):
                rounds[name].append(w.time_q32_rotated(name, time_calls, REPS))
            else:
                rounds[name].append(time_calls(lambda: w.run(name), torch, REPS))
    per = {name: statistics.median(v) for name, v in rounds.items()}
    step_input = sum(w.calls[c]["inp"] for c in STEP)
    value = step_input / (ms_per_step / 1e3) / 1e9
    log("step %.3f ms (wall %.3f ms/step)" % (ms_per_step, wall_ms / args.steps))

    detail = {}
    for name in STEP:
        ms = per[name]
        c = w.calls[name]
        detail[name] = dict(us=round(ms * 1e3, 2), input_gbs=round(c["inp"] / ms / 1e6, 1),
                            rw_gbs=round(c["rw"] / ms / 1e6, 1), pct_hbm_peak=round(100 * c["rw"] / ms / 1e6 / PEAK_GBS, 1))

    # Roofline of the dominant kernel: the slower (by its in-step launch time, from the event
    # spans of kernel_step_loop) of the data kernel inside bq_quantize_nested and the kernel of
    # bq_dequantize_nested.  The data kernel's algorithmic bytes are the method's: 2 B of bf16
    # read and 0.5 B of codes written per element; the 16-bit block maxima it also writes for
    # the statistics kernels (2 B per block) are reported as intermediate bytes.
    n = w.N5
    mean = statistics.fmean
    qk_mean, dk_mean = mean(q_sp) - mean(q8_sp), mean(d_sp) - mean(q4_sp)
    q_bytes = 2 * n + n // 2
    q_inter = 2 * w.nb
    dq_bytes = w.calls["dequantize_nested"]["rw"]
    us = lambda v: round(v * 1e3, 2)  # noqa: E731
    detail["quantize_nested data kernel (in-step, event spans)"] = dict(
        us=us(qk_mean), span_q8_q_us=us(mean(q_sp)), span_q8_us=us(mean(q8_sp)),
        pct_hbm_peak=round(100 * q_bytes / qk_mean / 1e6 / PEAK_GBS, 1),
        pct_hbm_peak_with_intermediate=round(100 * (q_bytes + q_inter) / qk_mean / 1e6 / PEAK_GBS, 1))
    detail["dequantize_nested kernel (in-step, event spans)"] = dict(
        us=us(dk_mean), span_d_q4_us=us(mean(d_sp)), span_q4_us=us(mean(q4_sp)),
        pct_hbm_peak=round(100 * dq_bytes / dk_mean / 1e6 / PEAK_GBS, 1))
    detail["quantize_blockwise of the same tensor (no statistics)"] = dict(
        us=round(per["quantize_kernel"] * 1e3, 2),
        pct_hbm_peak=round(100 * (q_bytes + 4 * w.nb) / per["quantize_kernel"] / 1e6 / PEAK_GBS, 1))
    if qk_mean >= dk_mean:
        roofline = dict(kernel="quantize_kernel<2, 4, 0, 1, true>, the data kernel of bq_quantize_nested",
                        bytes_per_launch=q_bytes, intermediate_bytes_per_launch=q_inter, ms=qk_mean,
                        traffic=traffic_for("quantize_kernel"))
    else:
        roofline = dict(kernel="dequantize_nested_kernel<2, 4>, the kernel of bq_dequantize_nested",
                        bytes_per_launch=dq_bytes, ms=dk_mean, traffic=traffic_for("dequantize_nested_kernel"))
    kms = roofline.pop("ms")
    achieved = roofline["bytes_per_launch"] / kms / 1e6
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_GBS, 4), traffic=roofline.pop("traffic"),
                    us_per_launch=round(kms * 1e3, 2), launches=len(q_sp), **roofline)

    if not args.no_detail:
        log("timing the individual workloads")
        detail.update(detail_configs(bq, synth, torch, dev, PEAK_GBS))
    cpu = parity = None
    if not args.no_cpu_baseline:
        log("running the CPU oracle on the step input (threaded), then a single-thread sample")
        cpu, parity = cpu_baseline_and_parity(w, torch, gpu_out)
        del gpu_out

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "bf16 2^29 (1 GiB) 4-bit blockwise B=64 nested-statistics quantize + dequantize, "
                               "plus GGUF-style 4096x14336 Q4 and Q8 block dequant to bf16",
                   "n": w.N5, "blocksize": w.B5, "blocksize2": w.B2, "gguf_shape": [w.ROWS, w.COLS],
                   "step_input_bytes": step_input},
        "roofline": roofline, "cpu_baseline": cpu, "parity": parity, "detail": detail,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
