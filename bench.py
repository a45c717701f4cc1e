"""Benchmark of the FP8 hot path on one MI355X.

One step = the forward pass of a 1.5B-class linear layer with hybrid-granularity
FP8 (token-wise 1x128 E4M3 activations, 128x128-block E4M3 weights, UE8M0
round-up scales) on seeded synthetic bf16 tensors already resident in HBM:
  1. fp8_quantize_token  X [4096 x 1536] bf16 -> codes + scales
  2. fp8_quantize_block  W [8960 x 1536] bf16 -> codes + scales
  3. fp8_block_scaled_gemm  Y = Xq * Wq^T, M=4096 N=8960 K=1536, fp32 accumulate, bf16 out
`value` is the whole step's throughput in TFLOP/s (2*M*N*K per step / step
time), with the step's launches captured once in a HIP graph and replayed
(the launches are asynchronous and allocate nothing, so a replay is the same
work without the host's per-launch cost).  In a separate eager pass each
entry point is timed with events on the stream it runs on, and the dominant
one (the GEMM) is reported against the dense FP8 MFMA peak.
`cpu_baseline` times the CPU oracle on a bounded sample of the same step.

Other workloads (--workload): dgrad7b, wgrad, mxfprop1p5b (the fprop step on
MX operands: 32-element E8M0 scales for X and W, mx_gemm), f32sfprop1p5b
(the fprop step with fp32 instead of power-of-two scales), dualq (the
two-orientation quantizers on the wgrad activation and the dgrad weight),
gaussws7b (GaussWS sampling of the dgrad weight from fp32 master weights),
mxstress -- for the per-kernel roofline figures; they print the same kind of
JSON line.  gemmsweep times the GEMM alone over N and K (M = 4096) and fits
the per-round fixed cost; copy times a plain 256 MiB device copy.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA, TFLOP/s
METRIC = "FP8 quantize GB/s + block-scaled FP8 GEMM TFLOP/s, % of MI355X peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="fprop1p5b",
                   choices=["fprop1p5b", "dgrad7b", "wgrad", "mxfprop1p5b", "f32sfprop1p5b", "dualq", "gaussws7b",
                            "mxstress", "copy", "gemmsweep"])
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-rows", type=int, default=0,
                   help="token rows in the oracle sample (0 = all rows: the full step)")
    return p.parse_args()


def to_dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


class KernelTimer:
    """Event pairs around each launch on the current stream; averages per kernel."""

    def __init__(self):
        self.pending = []
        self.times = {}

    def run(self, name, fn):
        import torch
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn()
        e.record()
        self.pending.append((name, s, e))
        return out

    def collect(self):
        for name, s, e in self.pending:
            self.times.setdefault(name, []).append(s.elapsed_time(e) * 1e-3)
        self.pending = []

    def mean(self, name):
        return float(np.mean(self.times[name]))

    def median(self, name):
        return float(np.median(self.times[name]))


class ColdTimer(KernelTimer):
    """Like KernelTimer, but every timed call is preceded by a write of a 512 MiB scrub
    buffer (twice the 256 MB last-level cache), outside the event pair: the call then
    finds none of its inputs in the caches."""

    def __init__(self, scrub):
        super().__init__()
        self.scrub = scrub
        self.count = 0

    def run(self, name, fn):
        self.count += 1
        self.scrub.fill_(self.count & 0xFF)
        return super().run(name, fn)


def context_measurements(step, timer, reps=10):
    """Median warm and cold (scrubbed) per-call times, the device description and a
    measured device copy bandwidth, added to the JSON line as context."""
    import torch
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = ColdTimer(scrub)
    step(cold)  # warm-up of the scrub path
    torch.cuda.synchronize()
    cold.pending = []
    for _ in range(reps):
        step(cold)
    torch.cuda.synchronize()
    cold.collect()
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(10):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 10 / (s.elapsed_time(e) * 1e-3) / 1e9
    del scrub, src, dst
    props = torch.cuda.get_device_properties(0)
    per = {name: {"us_median": round(timer.median(name) * 1e6, 2),
                  "us_cold_median": round(cold.median(name) * 1e6, 2)} for name in timer.times}
    return per, {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                 "compute_units": props.multi_processor_count, "copy_256MiB_GBs": round(copy_gbs, 1)}


def add_context(line, step, timer):
    per, device = context_measurements(step, timer)
    for name, d in per.items():
        if name in line["kernels"]:
            line["kernels"][name].update(d)
    line["device"] = device
    line["timing"] = ("value: replays of a graph of steps_per_graph whole steps between synchronisations; "
                      "kernels.us: mean of "
                      "event-bracketed eager calls inside the step (us_median: median); us_cold_median: each "
                      "call after a 512 MiB scrub write, medians of 10; roofline.achieved: from gemm.us; "
                      "gemm.us_back_to_back: mean of GEMM calls issued back to back between one event pair "
                      "(operands left in the caches by the previous call: context, not the step)")
    return line


class _NoTimer:
    def run(self, name, fn):
        return fn()


class _CaptureTimer(_NoTimer):
    """Runs a step and keeps each named launch's closure."""

    def __init__(self):
        self.fns = {}

    def run(self, name, fn):
        self.fns[name] = fn
        return fn()


def back_to_back(step, name, reps, warmup=3):
    """Mean seconds per call of the step's launch `name`, issued `reps` times back to back
    between one event pair on the current stream: the device never waits for the host
    between the calls, and each call finds its operands where the previous one left them
    in the caches (inside the step the quantizers' input streams evict them first).  The
    step runs once first, so the launch reads what the step's earlier launches wrote."""
    import torch
    cap = _CaptureTimer()
    step(cap)
    fn = cap.fns[name]
    for _ in range(warmup):
        _check(fn(), name)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def steps_per_graph(steps, cap=10):
    """Steps captured in one graph: the largest divisor of `steps` up to `cap`, so that
    whole replays cover exactly `steps` steps."""
    return max(d for d in range(1, min(cap, steps) + 1) if steps % d == 0)


def time_graph(step, steps, warmup, outputs):
    """Captures S consecutive steps in one HIP graph (S = steps_per_graph(steps): a
    replay of a graph launch costs the device an idle gap of ~8 us before its first
    kernel, which one step per graph would pay every step), checks that a replay
    reproduces the eager step's outputs bit for bit, then times steps / S replays
    (after warmup / S, rounded up) between device synchronisations.  Every step is the
    whole path on the same batch.  Returns (seconds per step, S)."""
    import torch
    steps = max(1, steps)
    per_graph = steps_per_graph(steps)
    step(_NoTimer())
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            step(_NoTimer())
    for o in outputs:
        o.zero_()
    g.replay()
    torch.cuda.synchronize()
    for o, r in zip(outputs, ref):
        if not torch.equal(o, r):
            raise RuntimeError("graph replay differs from the eager step")
    for _ in range(-(-warmup // per_graph)):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps // per_graph):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps, per_graph


def time_steps(step, steps, warmup):
    import torch
    timer = KernelTimer()
    for _ in range(warmup):
        step(timer)
    torch.cuda.synchronize()
    timer.pending = []
    timer.times = {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.collect()
    return wall / steps, timer


# ----------------------------------------------------------------------- workloads

def fprop_setup():
    import synth
    d = synth.fprop1p5b()
    return {"x": to_dev(d["x"]), "w": to_dev(d["w"]), "host": d}


def _check(st, what):
    if st != 0:
        raise RuntimeError("%s returned status %d" % (what, st))


def fprop_step_fn(t):
    """The step through the C-ABI entry points with outputs allocated once, so the events
    bracket exactly one entry point each.  Returns (step, outputs)."""
    import torch
    import mx_block_scaled_x128_amd as mx
    x, w = t["x"], t["w"]
    M, K = x.shape
    N = w.shape[0]
    dev = x.device
    xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    xs = torch.empty((M, K // 128), dtype=torch.uint8, device=dev)
    wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
    ws = torch.empty((N // 128, K // 128), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step(timer):
        stream = torch.cuda.current_stream().cuda_stream
        _check(timer.run("quant_token_x", lambda: mx.fp8_quantize_token(
            x.data_ptr(), mx.BF16, M, K, K, mx.ROW, mx.E4M3, xq.data_ptr(), K, xs.data_ptr(), stream)),
            "fp8_quantize_token")
        _check(timer.run("quant_block_w", lambda: mx.fp8_quantize_block(
            w.data_ptr(), mx.BF16, N, K, K, mx.E4M3, wq.data_ptr(), K, ws.data_ptr(), stream)),
            "fp8_quantize_block")
        _check(timer.run("gemm", lambda: mx.fp8_block_scaled_gemm(
            M, N, K, xq.data_ptr(), K, mx.E4M3, xs.data_ptr(), wq.data_ptr(), K, mx.E4M3, mx.B_NK,
            ws.data_ptr(), mx.SCALE_BLOCK128, y.data_ptr(), N, mx.BF16, stream)), "fp8_block_scaled_gemm")
    return step, [xq, xs, wq, ws, y]


def cpu_baseline_fprop(host, rows):
    """Oracle on a bounded sample: `rows` token rows of X through the token quantizer and
    the GEMM, plus the whole weight quantizer; scaled to the full step."""
    import oracle
    threads = min(16, os.cpu_count() or 1)
    x, w = host["x"], host["w"]
    M, K = x.shape
    N = w.shape[0]
    rows = M if rows <= 0 else min(rows, M)
    xs = np.ascontiguousarray(x[:rows])
    t0 = time.perf_counter()
    xq, xsc = oracle.quantize_rows(xs, oracle.E4M3, threads=threads)
    t1 = time.perf_counter()
    wq, wsc = oracle.quantize_block(w, oracle.E4M3, threads=threads)
    t2 = time.perf_counter()
    oracle.gemm(xq, xsc, oracle.E4M3, wq, wsc, oracle.E4M3, threads=threads)
    t3 = time.perf_counter()
    scale = M / float(rows)
    t_step = (t1 - t0) * scale + (t2 - t1) + (t3 - t2) * scale
    return {
        "value": round(2.0 * M * N * K / t_step / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
        "kind": "oracle",
        "sample": ("the full step" if rows == M else
                   "%d of %d token rows through token quantization and the GEMM, full weight quantization, "
                   "times scaled to the full step" % (rows, M))
                  + " (oracle: fp64 C, %d host threads; %.1f s measured, %.1f s per step)" % (threads, t3 - t0, t_step),
    }


def gemm_traffic(workload):
    """HBM bytes per GEMM call from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded
    under profiles/ (scaled by a plain copy's counters), or None when the GEMM kernel's
    source has changed since they were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    rec_path = os.path.join(here, "profiles", "gemm_traffic_%s.json" % workload)
    src = os.path.join(here, "mx_block_scaled_x128_amd", "csrc", "gemm.hip")
    if not os.path.exists(rec_path):
        return None
    rec = json.load(open(rec_path))
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec.get("gemm_source_sha256"):
        return None
    return int(rec["fetch_bytes_per_call"] + rec["write_bytes_per_call"])


def bytes_token(rows, cols, in_bytes):
    return rows * cols * (in_bytes + 1) + rows * ((cols + 127) // 128)


def bytes_block(rows, cols, in_bytes):
    return rows * cols * (in_bytes + 1) + ((rows + 127) // 128) * ((cols + 127) // 128)


def bench_fprop(args):
    import torch
    t = fprop_setup()
    M, K = t["x"].shape
    N = t["w"].shape[0]
    step, outputs = fprop_step_fn(t)
    per_step_eager, timer = time_steps(step, args.steps, args.warmup)
    per_step, per_graph = time_graph(step, args.steps, args.warmup, outputs)
    flops = 2.0 * M * N * K
    g = timer.mean("gemm")
    gb = back_to_back(step, "gemm", max(20, args.steps))
    qx = timer.mean("quant_token_x")
    qw = timer.mean("quant_block_w")
    bx = bytes_token(M, K, 2)
    bw = bytes_block(N, K, 2)
    gemm_tflops = flops / g / 1e12
    line = {
        "metric": METRIC, "value": round(flops / per_step / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(per_step * 1e3, 4),
        "ms_per_step_eager": round(per_step_eager * 1e3, 4), "steps_per_graph": per_graph,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3",
        "data": "synthetic (seeded numpy PCG64; bf16 inputs resident in HBM before timing)",
        "config": {"workload": "fprop1p5b: token-quantize X 4096x1536 bf16 (1x128, E4M3) + block-quantize "
                               "W 8960x1536 bf16 (128x128, E4M3) + block-scaled GEMM M=4096 N=8960 K=1536 "
                               "bf16 out", "M": M, "N": N, "K": K, "global_batch": M, "parallelism": "single GPU"},
        "kernels": {
            "quant_token_x": {"us": round(qx * 1e6, 2), "GB/s": round(bx / qx / 1e9, 1),
                              "frac_hbm_peak": round(bx / qx / 1e9 / HBM_PEAK_GBS, 4), "bytes": bx},
            "quant_block_w": {"us": round(qw * 1e6, 2), "GB/s": round(bw / qw / 1e9, 1),
                              "frac_hbm_peak": round(bw / qw / 1e9 / HBM_PEAK_GBS, 4), "bytes": bw},
            "gemm": {"us": round(g * 1e6, 2), "TFLOP/s": round(gemm_tflops, 1),
                     "frac_fp8_peak": round(gemm_tflops / FP8_PEAK_TFLOPS, 4), "flops": flops,
                     "us_back_to_back": round(gb * 1e6, 2)},
        },
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": gemm_traffic("fprop1p5b"),
                     "traffic_note": "HBM bytes per GEMM call (FETCH_SIZE + WRITE_SIZE, copy-calibrated; "
                                     "profiles/gemm_traffic_fprop1p5b.json); algorithmic bytes %d"
                                     % (M * K + N * K + M * (K // 128) + ((N + 127) // 128) * (K // 128)
                                        + 2 * M * N)},
    }
    add_context(line, step, timer)
    line["cpu_baseline"] = None if args.no_cpu else cpu_baseline_fprop(t["host"], args.cpu_rows)
    return line


def bench_gemm_sweep(args):
    """The block-scaled GEMM at M = 4096 over N and K, bf16 output (and fp32 output at one
    shape), uniformly random finite E4M3 codes with scale bytes in [120, 134]: one round of
    256x256 tiles at N = 4096 (256 tiles, one per CU), two rounds at N = 8192.  Per shape,
    `warmup` calls and then `steps` calls back to back between one event pair (mean per
    call).  A least-squares line through the one-round bf16 points, time = fixed + slope x
    (K / 128), separates the cost of a round that does not scale with K (prologue, output
    write) from the K loop."""
    import torch
    import mx_block_scaled_x128_amd as mx
    import synth
    M = 4096
    shapes = [(4096, 256, True), (4096, 512, True), (4096, 1536, True), (4096, 3072, True), (4096, 6144, True),
              (8192, 1536, True), (4096, 1536, False)]
    res = []
    for i, (N, K, bf16) in enumerate(shapes):
        a = torch.from_numpy(synth.random_codes(7000 + 4 * i, (M, K), 0)).cuda()
        b = torch.from_numpy(synth.random_codes(7001 + 4 * i, (N, K), 0)).cuda()
        sa = torch.from_numpy(synth.random_scale_bytes(7002 + 4 * i, (M, K // 128))).cuda()
        sb = torch.from_numpy(synth.random_scale_bytes(7003 + 4 * i, (N // 128, K // 128))).cuda()
        out = torch.empty((M, N), dtype=torch.bfloat16 if bf16 else torch.float32, device="cuda")

        def call():
            mx.block_scaled_gemm(a, sa, mx.E4M3, b, sb, mx.E4M3, mx.B_NK, mx.SCALE_BLOCK128, out=out)
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        res.append({"M": M, "N": N, "K": K, "out": "bf16" if bf16 else "fp32", "us": round(us, 2),
                    "TFLOP/s": round(2.0 * M * N * K / us / 1e6, 1)})
        del a, b, sa, sb, out
    one = [r for r in res if r["N"] == 4096 and r["out"] == "bf16"]
    x = np.array([r["K"] / 128.0 for r in one])
    y = np.array([r["us"] for r in one])
    slope, fixed = np.polyfit(x, y, 1)
    best = max(res, key=lambda r: r["TFLOP/s"])
    return {"metric": "block-scaled FP8 GEMM TFLOP/s over N and K (M = 4096)", "value": best["TFLOP/s"],
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(best["us"] / 1e3, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic (random finite codes)",
            "config": {"workload": "gemmsweep: M=4096, N in {4096, 8192}, K in {256 .. 6144}"},
            "sweep": res, "fit_one_round_bf16": {"fixed_us": round(float(fixed), 2),
                                                 "us_per_k_block": round(float(slope), 3)},
            "roofline": {"bound": "mfma", "achieved": best["TFLOP/s"], "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(best["TFLOP/s"] / FP8_PEAK_TFLOPS, 4), "traffic": None},
            "cpu_baseline": None}


def bench_copy(args):
    """A plain device copy of 256 MiB (torch's copy kernel): the reference point that scales
    profiler byte counters (FETCH_SIZE / WRITE_SIZE) to bytes, and a measured bandwidth."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    per_step, timer = time_steps(lambda timer: timer.run("copy", lambda: dst.copy_(src)), args.steps, args.warmup)
    t = timer.mean("copy")
    return {"metric": "device copy GB/s (read + write)", "value": round(2 * n / t / 1e9, 1), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(per_step * 1e3, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "copy 256 MiB", "bytes_read": n, "bytes_written": n}, "roofline": None,
            "cpu_baseline": None}


def bench_other(args):
    """Per-kernel figures for the larger workloads (same JSON shape, kernels block filled).
    Outputs are allocated once; events bracket one C-ABI launch each."""
    import torch
    import mx_block_scaled_x128_amd as mx
    import synth
    u8 = dict(dtype=torch.uint8, device="cuda")

    def cur():
        return torch.cuda.current_stream().cuda_stream
    kern = {}
    if args.workload == "dgrad7b":
        d = synth.dgrad7b()
        dy, w = to_dev(d["dy"]), to_dev(d["w"])
        del d
        M, K = dy.shape
        N = w.shape[1]
        gq, gs = torch.empty((M, K), **u8), torch.empty((M, K // 128), **u8)
        wq, ws = torch.empty((K, N), **u8), torch.empty((K // 128, N // 128), **u8)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def step(timer):
            stream = cur()
            _check(timer.run("quant_token_dy", lambda: mx.fp8_quantize_token(
                dy.data_ptr(), mx.BF16, M, K, K, mx.ROW, mx.E5M2, gq.data_ptr(), K, gs.data_ptr(), stream)), "q")
            _check(timer.run("quant_block_w", lambda: mx.fp8_quantize_block(
                w.data_ptr(), mx.BF16, K, N, N, mx.E4M3, wq.data_ptr(), N, ws.data_ptr(), stream)), "q")
            _check(timer.run("gemm", lambda: mx.fp8_block_scaled_gemm(
                M, N, K, gq.data_ptr(), K, mx.E5M2, gs.data_ptr(), wq.data_ptr(), N, mx.E4M3, mx.B_KN,
                ws.data_ptr(), mx.SCALE_BLOCK128, y.data_ptr(), N, mx.BF16, stream)), "gemm")
        sizes = {"quant_token_dy": bytes_token(M, K, 2), "quant_block_w": bytes_block(K, N, 2)}
        outputs = [gq, gs, wq, ws, y]
        flops = 2.0 * M * N * K
        desc = "dgrad7b: token-quantize dY 8192x18944 bf16 (E5M2) + block-quantize W 18944x3584 (E4M3) + GEMM " \
               "M=8192 N=3584 K=18944 (B stored [K][N]) bf16 out"
    elif args.workload == "wgrad":
        d = synth.wgrad()
        x, dy = to_dev(d["x"]), to_dev(d["dy"])
        del d
        T, C = x.shape
        xq, xs = torch.empty((C, T), **u8), torch.empty((C, T // 128), **u8)
        gq, gs = torch.empty((C, T), **u8), torch.empty((C, T // 128), **u8)
        y = torch.empty((C, C), dtype=torch.float32, device="cuda")

        def step(timer):
            stream = cur()
            _check(timer.run("quant_col_x", lambda: mx.fp8_quantize_token(
                x.data_ptr(), mx.BF16, T, C, C, mx.COL_T, mx.E4M3, xq.data_ptr(), T, xs.data_ptr(), stream)), "q")
            _check(timer.run("quant_col_dy", lambda: mx.fp8_quantize_token(
                dy.data_ptr(), mx.BF16, T, C, C, mx.COL_T, mx.E5M2, gq.data_ptr(), T, gs.data_ptr(), stream)), "q")
            _check(timer.run("gemm", lambda: mx.fp8_block_scaled_gemm(
                C, C, T, gq.data_ptr(), T, mx.E5M2, gs.data_ptr(), xq.data_ptr(), T, mx.E4M3, mx.B_NK,
                xs.data_ptr(), mx.SCALE_ROW128, y.data_ptr(), C, mx.F32, stream)), "gemm")
        sizes = {"quant_col_x": bytes_token(T, C, 2), "quant_col_dy": bytes_token(T, C, 2)}
        outputs = [xq, xs, gq, gs, y]
        M = N = C
        K = T
        flops = 2.0 * M * N * K
        desc = "wgrad: column-quantize X and dY 16384x4096 bf16 along tokens (E4M3 / E5M2) + GEMM M=N=4096 " \
               "K=16384 fp32 out"
    elif args.workload == "mxfprop1p5b":
        d = synth.fprop1p5b()
        x, w = to_dev(d["x"]), to_dev(d["w"])
        del d
        M, K = x.shape
        N = w.shape[0]
        xq, xs = torch.empty((M, K), **u8), torch.empty((M, K // 32), **u8)
        wq, ws = torch.empty((N, K), **u8), torch.empty((N, K // 32), **u8)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def step(timer):
            stream = cur()
            _check(timer.run("mx_quant_x", lambda: mx.mx_quantize(
                x.data_ptr(), mx.BF16, M, K, K, mx.E4M3, mx.RULE_FLOOR, xq.data_ptr(), K, xs.data_ptr(), None,
                stream)), "mx")
            _check(timer.run("mx_quant_w", lambda: mx.mx_quantize(
                w.data_ptr(), mx.BF16, N, K, K, mx.E4M3, mx.RULE_FLOOR, wq.data_ptr(), K, ws.data_ptr(), None,
                stream)), "mx")
            _check(timer.run("gemm", lambda: mx.mx_gemm(
                M, N, K, xq.data_ptr(), K, mx.E4M3, xs.data_ptr(), wq.data_ptr(), K, mx.E4M3, ws.data_ptr(),
                y.data_ptr(), N, mx.BF16, stream)), "gemm")
        sizes = {"mx_quant_x": M * K * 3 + M * K // 32, "mx_quant_w": N * K * 3 + N * K // 32}
        outputs = [xq, xs, wq, ws, y]
        flops = 2.0 * M * N * K
        desc = "mxfprop1p5b: MX-quantize X 4096x1536 and W 8960x1536 bf16 (32-element E4M3 blocks, OCP floor " \
               "scales) + MX GEMM M=4096 N=8960 K=1536 bf16 out"
    elif args.workload == "f32sfprop1p5b":
        d = synth.fprop1p5b()
        x, w = to_dev(d["x"]), to_dev(d["w"])
        del d
        M, K = x.shape
        N = w.shape[0]
        f32 = dict(dtype=torch.float32, device="cuda")
        xq, xs = torch.empty((M, K), **u8), torch.empty((M, K // 128), **f32)
        wq, ws = torch.empty((N, K), **u8), torch.empty(((N + 127) // 128, K // 128), **f32)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def step(timer):
            stream = cur()
            _check(timer.run("quant_token_x_f32s", lambda: mx.fp8_quantize_token_f32s(
                x.data_ptr(), mx.BF16, M, K, K, mx.ROW, mx.E4M3, xq.data_ptr(), K, xs.data_ptr(), stream)), "q")
            _check(timer.run("quant_block_w_f32s", lambda: mx.fp8_quantize_block_f32s(
                w.data_ptr(), mx.BF16, N, K, K, mx.E4M3, wq.data_ptr(), K, ws.data_ptr(), stream)), "q")
            _check(timer.run("gemm", lambda: mx.fp8_gemm_f32s(
                M, N, K, xq.data_ptr(), K, mx.E4M3, xs.data_ptr(), wq.data_ptr(), K, mx.E4M3, mx.B_NK,
                ws.data_ptr(), mx.SCALE_BLOCK128, y.data_ptr(), N, mx.BF16, stream)), "gemm")
        sizes = {"quant_token_x_f32s": M * K * 3 + 4 * M * (K // 128),
                 "quant_block_w_f32s": N * K * 3 + 4 * ((N + 127) // 128) * (K // 128)}
        outputs = [xq, xs, wq, ws, y]
        flops = 2.0 * M * N * K
        desc = "f32sfprop1p5b: token-quantize X 4096x1536 and block-quantize W 8960x1536 bf16 with fp32 scales " \
               "(amax / 448) + GEMM over fp32-scaled operands M=4096 N=8960 K=1536 bf16 out"
    elif args.workload == "gaussws7b":
        wf = synth.bf16_bits_to_f32(synth.dgrad7b(rows=16)["w"]).astype(np.float32)
        R, C = wf.shape
        bt_np = np.random.default_rng(10).integers(4, 9, (-(-R // 32), -(-C // 32))).astype(np.int8)
        w = to_dev(wf)
        bt = torch.from_numpy(bt_np).cuda()
        del wf
        w_hat = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
        counter = [0]

        def step(timer):
            stream = cur()
            _check(timer.run("gaussws", lambda: mx.gaussws_sample(
                w.data_ptr(), mx.F32, R, C, C, bt.data_ptr(), 2025, 7, w_hat.data_ptr(), C, stream)), "gws")
        sizes = {"gaussws": R * C * 6 + bt_np.size}
        outputs = [w_hat]
        flops = 0.0
        M = N = K = 0
        desc = "gaussws7b: GaussWS sampled weight of W 18944x3584 fp32 master weights (32x32 blocks, int8 " \
               "bitwidths 4..8, Philox4x64-10 rounded-normal noise) -> bf16"
    elif args.workload == "dualq":
        x = to_dev(synth.wgrad()["x"])
        w = to_dev(synth.dgrad7b(rows=16)["w"])
        T, C = x.shape
        O, I = w.shape
        xq, xs = torch.empty((T, C), **u8), torch.empty((T, C // 128), **u8)
        xqt, xst = torch.empty((C, T), **u8), torch.empty((C, T // 128), **u8)
        wq, ws = torch.empty((O, I), **u8), torch.empty(((O + 127) // 128, I // 128), **u8)
        wqt, wst = torch.empty((I, O), **u8), torch.empty((I // 128, (O + 127) // 128), **u8)

        def step(timer):
            stream = cur()
            _check(timer.run("token_dual_x", lambda: mx.fp8_quantize_token_dual(
                x.data_ptr(), mx.BF16, T, C, C, mx.E4M3, xq.data_ptr(), C, xs.data_ptr(), xqt.data_ptr(), T,
                xst.data_ptr(), stream)), "dual")
            _check(timer.run("block_dual_w", lambda: mx.fp8_quantize_block_dual(
                w.data_ptr(), mx.BF16, O, I, I, mx.E4M3, wq.data_ptr(), I, ws.data_ptr(), wqt.data_ptr(), O,
                wst.data_ptr(), stream)), "dual")
        sizes = {"token_dual_x": T * C * 4 + 2 * T * C // 128,
                 "block_dual_w": O * I * 4 + 2 * ((O + 127) // 128) * (I // 128)}
        outputs = [xq, xs, xqt, xst, wq, ws, wqt, wst]
        flops = 0.0
        M = N = K = 0
        desc = "dualq: X 16384x4096 bf16 -> 1x128 row codes + 128-token column codes (transposed), one read; " \
               "W 18944x3584 bf16 -> 128x128 block codes + their transpose"
    else:
        xs_ = [to_dev(synth.mxstress_tensor(j)) for j in range(64)]
        R, C = xs_[0].shape
        q, sc, cn = torch.empty((R, C), **u8), torch.empty((R, C // 32), **u8), torch.empty((R, C // 32), **u8)

        def step(timer):
            stream = cur()
            for j in range(64):
                _check(timer.run("mx_quant", lambda: mx.mx_quantize(
                    xs_[j].data_ptr(), mx.F32, R, C, C, mx.E4M3, mx.RULE_FLOOR, q.data_ptr(), C, sc.data_ptr(),
                    cn.data_ptr(), stream)), "mx")
        sizes = {"mx_quant": R * C * 5 + 2 * R * (C // 32)}
        outputs = [q, sc, cn]
        flops = 0.0
        M = N = K = 0
        desc = "mxstress: 64 tensors 4096x4096 fp32, MX 32-element E4M3 blocks, OCP floor scales, clamp counts"
    per_step_eager, timer = time_steps(step, args.steps, args.warmup)
    per_step, per_graph = time_graph(step, args.steps, args.warmup, outputs)
    for name, b in sizes.items():
        t = timer.mean(name)
        kern[name] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                      "frac_hbm_peak": round(b / t / 1e9 / HBM_PEAK_GBS, 4), "bytes": b}
    if flops:
        g = timer.mean("gemm")
        gb = back_to_back(step, "gemm", max(20, args.steps))
        kern["gemm"] = {"us": round(g * 1e6, 2), "TFLOP/s": round(flops / g / 1e12, 1),
                        "frac_fp8_peak": round(flops / g / 1e12 / FP8_PEAK_TFLOPS, 4), "flops": flops,
                        "us_back_to_back": round(gb * 1e6, 2)}
        value, unit = flops / per_step / 1e12, "TFLOP/s"
        roof = {"bound": "mfma", "achieved": round(flops / g / 1e12, 2), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(flops / g / 1e12 / FP8_PEAK_TFLOPS, 4), "traffic": None}
    else:
        tot = sum(sizes.values()) * (64 if args.workload == "mxstress" else 1)
        value, unit = tot / per_step / 1e9, "GB/s"
        dom = max(sizes, key=lambda k: kern[k]["us"])
        roof = {"bound": "hbm", "achieved": kern[dom]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": kern[dom]["frac_hbm_peak"], "traffic": None, "kernel": dom}
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(per_step * 1e3, 4),
        "ms_per_step_eager": round(per_step_eager * 1e3, 4), "steps_per_graph": per_graph,
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8", "data": "synthetic (seeded numpy PCG64)",
        "config": {"workload": desc, "M": M, "N": N, "K": K}, "kernels": kern, "roofline": roof,
        "cpu_baseline": None,
    }
    if args.workload != "mxstress":  # 64 launches per step: the scrubbed pass would take long
        add_context(line, step, timer)
    return line


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (requested --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import mx_block_scaled_x128_amd as mx
    mx.load_library()  # fail loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.workload == "fprop1p5b":
        line = bench_fprop(args)
    elif args.workload == "copy":
        line = bench_copy(args)
    elif args.workload == "gemmsweep":
        line = bench_gemm_sweep(args)
    else:
        line = bench_other(args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
