"""Benchmark of the FP8 hot path on one MI355X.

Default step (workload dgrad7b): the input-gradient pass of a 7B-class linear
layer with hybrid-granularity FP8, on seeded synthetic bf16 tensors already
resident in HBM:
  1. fp8_quantize_token  dY [8192 x 18944] bf16 -> 1x128 E5M2 codes + E8M0 scales
  2. fp8_quantize_block  W [18944 x 3584] bf16 -> 128x128 E4M3 codes + E8M0 scales
  3. fp8_block_scaled_gemm  dX = dYq * Wq, M=8192 N=3584 K=18944 (W stored [K][N]),
     fp32 accumulation, bf16 out
`value` is the whole step's throughput in TFLOP/s (2*M*N*K per step / step time),
with the steps' asynchronous calls enqueued back to back between two device
synchronisations.  In a second pass each entry point is timed with events on the
stream it runs on, and the dominant one (the GEMM) is reported against the dense
FP8 MFMA peak (`roofline`).  The same steps replayed from a captured HIP graph are
reported as context (the calls allocate and synchronise nothing, so they capture).
`cpu_baseline` times the CPU oracle on a bounded sample of the same step.

Other workloads (--workload) print the same kind of line: fprop1p5b (forward of
a 1.5B-class layer), wgrad (weight gradient from column-quantized activations and
gradients), mxfprop1p5b (the forward on MX operands: 32-element E8M0 scales,
mx_gemm), f32sfprop1p5b (the forward with fp32 instead of power-of-two scales),
dualq (the two-orientation quantizers), gaussws7b (GaussWS sampling of the 7B
weight from fp32 master weights), mxstress (MX quantization with clamp counts of
64 distinct 4096x4096 fp32 tensors, with the clamp statistics).  gemmsweep times
the GEMM alone over N and K; vendorgemm times the GEMM beside the FP8 products
of the ROCm BLAS library (torch._scaled_mm) on the same shapes; copy times a
plain 256 MiB device copy.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
                       [--cpu-rows R]
"""
import argparse
import contextlib
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA, TFLOP/s
METRIC = "FP8 quantize GB/s + block-scaled FP8 GEMM TFLOP/s, % of MI355X peak"
HERE = os.path.dirname(os.path.abspath(__file__))
WORKLOADS = ["dgrad7b", "fprop1p5b", "wgrad", "mxfprop1p5b", "f32sfprop1p5b", "dualq", "gaussws7b", "mxstress",
             "copy", "gemmsweep", "vendorgemm"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="dgrad7b", choices=WORKLOADS)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-rows", type=int, default=-1,
                   help="output rows of the GEMM in the oracle sample (0 = all; default: per workload)")
    return p.parse_args()


def to_dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def oracle_threads():
    """Host threads for the oracle: the machine's cores, at most 16 (a one-GPU share of
    a multi-GPU host's cores)."""
    return min(16, os.cpu_count() or 1)


def _check(st, what):
    if st != 0:
        raise RuntimeError("%s returned status %d" % (what, st))


# ------------------------------------------------------------------------ timing

class KernelTimer:
    """Event pairs around each launch on the current stream; averages per kernel.  The
    events come from a pool made (and recorded once) in advance, so that a timed call
    costs the host two event records and the launch: the host stays ahead of the device,
    and an event pair does not span a wait for the host."""

    def __init__(self):
        self.pending = []
        self.times = {}
        self.pool = []

    def reserve(self, n):
        import torch
        while len(self.pool) < n:
            e = torch.cuda.Event(enable_timing=True)
            e.record()  # creates the device event now
            self.pool.append(e)

    def _event(self):
        import torch
        return self.pool.pop() if self.pool else torch.cuda.Event(enable_timing=True)

    def run(self, name, fn):
        s, e = self._event(), self._event()
        s.record()
        out = fn()
        e.record()
        self.pending.append((name, s, e, 1))
        return out

    def run_many(self, name, fns):
        """Launches of one kernel issued back to back inside one event pair; each
        counts as the pair's time divided by their number (a pair per launch would
        measure the host when it issues launches slower than the device runs them)."""
        s, e = self._event(), self._event()
        s.record()
        outs = [fn() for fn in fns]
        e.record()
        self.pending.append((name, s, e, len(fns)))
        return outs

    def collect(self):
        for name, s, e, n in self.pending:
            self.times.setdefault(name, []).extend([s.elapsed_time(e) * 1e-3 / n] * n)
            self.pool += [s, e]
        self.pending = []

    def mean(self, name):
        return float(np.mean(self.times[name]))

    def median(self, name):
        return float(np.median(self.times[name]))


class ColdTimer(KernelTimer):
    """Like KernelTimer, but every timed call is preceded, outside the event pair, by a
    pass over a 512 MiB scrub buffer (twice the 256 MB last-level cache), so that the
    call finds none of its inputs in the caches.  A read pass (`dirty=False`) leaves the
    caches full of clean lines; a write pass leaves them full of dirty ones, which the
    memory system writes back while the timed call runs (its time then includes the
    write-back of the scrub's own data)."""

    def __init__(self, scrub, dirty=False):
        import torch
        super().__init__()
        self.scrub = scrub
        self.dirty = dirty
        self.count = 0
        self.words = scrub.view(torch.int64)
        self.acc = torch.zeros(1, dtype=torch.int64, device=scrub.device)

    def _scrub(self):
        import torch
        self.count += 1
        if self.dirty:
            self.scrub.fill_(self.count & 0xFF)
        else:
            torch.sum(self.words.view(1, -1), dim=1, out=self.acc)

    def run(self, name, fn):
        self._scrub()
        return super().run(name, fn)

    def run_many(self, name, fns):
        self._scrub()  # once, before the batch
        return super().run_many(name, fns)


class _NoTimer:
    def run(self, name, fn):
        return fn()

    def run_many(self, name, fns):
        return [fn() for fn in fns]


class _CaptureTimer(_NoTimer):
    """Runs a step and keeps each named launch's closure."""

    def __init__(self):
        self.fns = {}

    def run(self, name, fn):
        self.fns[name] = fn
        return fn()

    def run_many(self, name, fns):
        self.fns[name] = fns[-1]
        return [fn() for fn in fns]


def context_measurements(step, timer, reps=10):
    """Median warm and cold (scrubbed: clean, then dirty caches) per-call times, the
    device description and a measured device copy bandwidth, added to the JSON line
    as context."""
    import torch
    scrub = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    colds = []
    for dirty in (False, True):
        cold = ColdTimer(scrub, dirty)
        step(cold)  # warm-up of the scrub path
        torch.cuda.synchronize()
        cold.pending = []
        for _ in range(reps):
            step(cold)
        torch.cuda.synchronize()
        cold.collect()
        colds.append(cold)
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
                  "us_cold_median": round(colds[0].median(name) * 1e6, 2),
                  "us_cold_dirty_median": round(colds[1].median(name) * 1e6, 2)} for name in timer.times}
    return per, {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                 "compute_units": props.multi_processor_count, "copy_256MiB_GBs": round(copy_gbs, 1)}


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


def ramp(step, min_seconds=0.3, min_steps=1):
    """Untimed steps until the device has been busy for min_seconds (and at least
    min_steps): the GPU raises its clock over the first tens of milliseconds of
    sustained load (measured on the dgrad step: the first ~40 steps run the GEMM 5-85 %
    slower than the steady ~410 us), which a few warmup steps after an idle host phase
    do not cover.  Returns the number of steps run."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while n < min_steps or time.perf_counter() - t0 < min_seconds:
        for _ in range(4):
            step(_NoTimer())
        n += 4
        torch.cuda.synchronize()
    return n


def time_plain(step, steps, warmup):
    """`warmup` untimed steps, then `steps` steps launched back to back from Python
    between two device synchronisations, with nothing else on the stream: the host
    enqueues the asynchronous calls far faster than the device runs them, so the wall
    time is the device's time for the step (Python's garbage collector is held off
    meanwhile).  Returns seconds per step."""
    import torch
    for _ in range(warmup):
        step(_NoTimer())
    torch.cuda.synchronize()
    with gc_paused():
        t0 = time.perf_counter()
        for _ in range(steps):
            step(_NoTimer())
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    return wall / steps


def time_steps(step, steps, warmup):
    """The eager pass with events: `steps` steps launched from Python, each entry point
    between an event pair (from the timer's pool), with Python's garbage collector held
    off during the pass (a collection pause while the device waits for the next launch
    would count as kernel time).  Returns (seconds per step, timer)."""
    import torch
    timer = KernelTimer()
    step(timer)  # a warm-up step that counts the step's launches
    timer.reserve(2 * len(timer.pending) * (warmup + steps))
    timer.pending = []
    for _ in range(warmup):
        step(timer)
    torch.cuda.synchronize()
    timer.pending = []
    timer.times = {}
    with gc_paused():
        t0 = time.perf_counter()
        for _ in range(steps):
            step(timer)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    timer.collect()
    return wall / steps, timer


@contextlib.contextmanager
def gc_paused():
    """Python's garbage collector off inside the block (no collection first: a pause
    of the host before the timed steps would leave the device idle long enough to
    lower its clock)."""
    was = gc.isenabled()
    gc.disable()
    try:
        yield
    finally:
        if was:
            gc.enable()


def recorded_traffic(workload):
    """HBM bytes per call of the dominant kernel from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs recorded under profiles/traffic_<workload>.json (scaled by a plain
    copy's counters), or None when the kernel's source file has changed since."""
    rec_path = os.path.join(HERE, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(rec_path):
        return None
    rec = json.load(open(rec_path))
    src = os.path.join(HERE, "mx_block_scaled_x128_amd", "csrc", rec["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return int(rec["fetch_bytes_per_call"] + rec["write_bytes_per_call"])


def bytes_token(rows, cols, in_bytes):
    return rows * cols * (in_bytes + 1) + rows * ((cols + 127) // 128)


def bytes_block(rows, cols, in_bytes):
    return rows * cols * (in_bytes + 1) + ((rows + 127) // 128) * ((cols + 127) // 128)


def cpu_line(value, unit, threads, seconds, sample):
    return {"value": round(value, 6), "unit": unit, "cores": threads, "host_cores": os.cpu_count(),
            "kind": "oracle",
            "sample": sample + " (oracle: fp64 C, %d host threads; %.1f s measured)" % (threads, seconds)}


# ----------------------------------------------------------------------- workloads
#
# Each workload builds its device tensors and returns a dict:
#   step(timer)  the whole path once, one named C-ABI call per timer.run
#   outputs      tensors a replay must reproduce bit for bit
#   sizes        algorithmic bytes per call of each quantizer launch
#   flops        2*M*N*K of the GEMM (0 when the step has none)
#   desc, config the workload description
#   cpu(rows)    the oracle on a bounded sample of the same step -> cpu_baseline

def w_dgrad7b():
    import torch
    import mx_block_scaled_x128_amd as mx
    import synth
    d = synth.dgrad7b()
    dy, w = to_dev(d["dy"]), to_dev(d["w"])
    M, K = dy.shape
    N = w.shape[1]
    u8 = dict(dtype=torch.uint8, device="cuda")
    gq, gs = torch.empty((M, K), **u8), torch.empty((M, K // 128), **u8)
    wq, ws = torch.empty((K, N), **u8), torch.empty((K // 128, N // 128), **u8)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step(timer):
        stream = torch.cuda.current_stream().cuda_stream
        _check(timer.run("quant_token_dy", lambda: mx.fp8_quantize_token(
            dy.data_ptr(), mx.BF16, M, K, K, mx.ROW, mx.E5M2, gq.data_ptr(), K, gs.data_ptr(), stream)),
            "fp8_quantize_token")
        _check(timer.run("quant_block_w", lambda: mx.fp8_quantize_block(
            w.data_ptr(), mx.BF16, K, N, N, mx.E4M3, wq.data_ptr(), N, ws.data_ptr(), stream)),
            "fp8_quantize_block")
        _check(timer.run("gemm", lambda: mx.fp8_block_scaled_gemm(
            M, N, K, gq.data_ptr(), K, mx.E5M2, gs.data_ptr(), wq.data_ptr(), N, mx.E4M3, mx.B_KN,
            ws.data_ptr(), mx.SCALE_BLOCK128, y.data_ptr(), N, mx.BF16, stream)), "fp8_block_scaled_gemm")

    def cpu(rows):
        import oracle
        th = oracle_threads()
        rows = M if rows == 0 else min(rows if rows > 0 else 2048, M)
        t0 = time.perf_counter()
        q, s = oracle.quantize_rows(np.ascontiguousarray(d["dy"][:rows]), oracle.E5M2, threads=th)
        t1 = time.perf_counter()
        wq_, ws_ = oracle.quantize_block(d["w"], oracle.E4M3, threads=th)
        t2 = time.perf_counter()
        oracle.gemm(q, s, oracle.E5M2, wq_, ws_, oracle.E4M3, oracle.B_KN, oracle.B_SCALE_BLOCK, threads=th)
        t3 = time.perf_counter()
        f = M / float(rows)
        t_step = (t1 - t0) * f + (t2 - t1) + (t3 - t2) * f
        return cpu_line(2.0 * M * N * K / t_step / 1e12, "TFLOP/s", th, t3 - t0,
                        ("the full step" if rows == M else
                         "%d of %d rows of dY through token quantization and the GEMM, the whole weight "
                         "through block quantization, times scaled to the full step (%.1f s per step)"
                         % (rows, M, t_step)))
    return {"step": step, "outputs": [gq, gs, wq, ws, y],
            "sizes": {"quant_token_dy": bytes_token(M, K, 2), "quant_block_w": bytes_block(K, N, 2)},
            "flops": 2.0 * M * N * K, "M": M, "N": N, "K": K, "dtype": "fp8_e5m2 x fp8_e4m3",
            "gemm_bytes": M * K + K * N + M * (K // 128) + (K // 128) * (N // 128) + 2 * M * N,
            "desc": "dgrad7b: token-quantize dY 8192x18944 bf16 (1x128, E5M2) + block-quantize W 18944x3584 "
                    "bf16 (128x128, E4M3) + block-scaled GEMM dX = dY*W, M=8192 N=3584 K=18944 (W stored "
                    "[K][N]) bf16 out",
            "cpu": cpu}


def w_fprop1p5b():
    import torch
    import mx_block_scaled_x128_amd as mx
    import synth
    d = synth.fprop1p5b()
    x, w = to_dev(d["x"]), to_dev(d["w"])
    M, K = x.shape
    N = w.shape[0]
    u8 = dict(dtype=torch.uint8, device="cuda")
    xq, xs = torch.empty((M, K), **u8), torch.empty((M, K // 128), **u8)
    wq, ws = torch.empty((N, K), **u8), torch.empty((N // 128, K // 128), **u8)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

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

    def cpu(rows):
        import oracle
        th = oracle_threads()
        rows = M if rows <= 0 else min(rows, M)
        t0 = time.perf_counter()
        q, s = oracle.quantize_rows(np.ascontiguousarray(d["x"][:rows]), oracle.E4M3, threads=th)
        t1 = time.perf_counter()
        wq_, ws_ = oracle.quantize_block(d["w"], oracle.E4M3, threads=th)
        t2 = time.perf_counter()
        oracle.gemm(q, s, oracle.E4M3, wq_, ws_, oracle.E4M3, threads=th)
        t3 = time.perf_counter()
        f = M / float(rows)
        t_step = (t1 - t0) * f + (t2 - t1) + (t3 - t2) * f
        return cpu_line(2.0 * M * N * K / t_step / 1e12, "TFLOP/s", th, t3 - t0,
                        "the full step" if rows == M else
                        "%d of %d token rows, times scaled to the full step" % (rows, M))
    return {"step": step, "outputs": [xq, xs, wq, ws, y],
            "sizes": {"quant_token_x": bytes_token(M, K, 2), "quant_block_w": bytes_block(N, K, 2)},
            "flops": 2.0 * M * N * K, "M": M, "N": N, "K": K, "dtype": "fp8_e4m3",
            "gemm_bytes": M * K + N * K + M * (K // 128) + (N // 128) * (K // 128) + 2 * M * N,
            "desc": "fprop1p5b: token-quantize X 4096x1536 bf16 (1x128, E4M3) + block-quantize W 8960x1536 bf16 "
                    "(128x128, E4M3) + block-scaled GEMM M=4096 N=8960 K=1536 bf16 out",
            "cpu": cpu}


def w_wgrad():
    import torch
    import mx_block_scaled_x128_amd as mx
    import synth
    d = synth.wgrad()
    x, dy = to_dev(d["x"]), to_dev(d["dy"])
    T, C = x.shape
    u8 = dict(dtype=torch.uint8, device="cuda")
    xq, xs = torch.empty((C, T), **u8), torch.empty((C, T // 128), **u8)
    gq, gs = torch.empty((C, T), **u8), torch.empty((C, T // 128), **u8)
    y = torch.empty((C, C), dtype=torch.float32, device="cuda")

    def step(timer):
        stream = torch.cuda.current_stream().cuda_stream
        _check(timer.run("quant_col_x", lambda: mx.fp8_quantize_token(
            x.data_ptr(), mx.BF16, T, C, C, mx.COL_T, mx.E4M3, xq.data_ptr(), T, xs.data_ptr(), stream)), "q")
        _check(timer.run("quant_col_dy", lambda: mx.fp8_quantize_token(
            dy.data_ptr(), mx.BF16, T, C, C, mx.COL_T, mx.E5M2, gq.data_ptr(), T, gs.data_ptr(), stream)), "q")
        _check(timer.run("gemm", lambda: mx.fp8_block_scaled_gemm(
            C, C, T, gq.data_ptr(), T, mx.E5M2, gs.data_ptr(), xq.data_ptr(), T, mx.E4M3, mx.B_NK,
            xs.data_ptr(), mx.SCALE_ROW128, y.data_ptr(), C, mx.F32, stream)), "gemm")

    def cpu(rows):
        import oracle
        th = oracle_threads()
        rows = C if rows == 0 else min(rows if rows > 0 else 1024, C)
        t0 = time.perf_counter()
        xq_, xs_ = oracle.quantize_cols_t(d["x"], oracle.E4M3, threads=th)
        gq_, gs_ = oracle.quantize_cols_t(d["dy"], oracle.E5M2, threads=th)
        t1 = time.perf_counter()
        oracle.gemm(gq_[:rows], gs_[:rows], oracle.E5M2, xq_, xs_, oracle.E4M3, oracle.B_NK, oracle.B_SCALE_ROW,
                    threads=th)
        t2 = time.perf_counter()
        t_step = (t1 - t0) + (t2 - t1) * C / float(rows)
        return cpu_line(2.0 * C * C * T / t_step / 1e12, "TFLOP/s", th, t2 - t0,
                        "the full step" if rows == C else
                        "both column quantizations in full, %d of %d output rows of the GEMM, times scaled to "
                        "the full step (%.1f s per step)" % (rows, C, t_step))
    return {"step": step, "outputs": [xq, xs, gq, gs, y],
            "sizes": {"quant_col_x": bytes_token(T, C, 2), "quant_col_dy": bytes_token(T, C, 2)},
            "flops": 2.0 * C * C * T, "M": C, "N": C, "K": T, "dtype": "fp8_e5m2 x fp8_e4m3",
            "gemm_bytes": 2 * C * T + 2 * C * (T // 128) + 4 * C * C,
            "desc": "wgrad: column-quantize X and dY 16384x4096 bf16 along tokens (E4M3 / E5M2) + GEMM "
                    "dW = dY^T X, M=N=4096 K=16384 fp32 out",
            "cpu": cpu}


def w_mxfprop1p5b():
    import torch
    import mx_block_scaled_x128_amd as mx
    import synth
    d = synth.fprop1p5b()
    x, w = to_dev(d["x"]), to_dev(d["w"])
    M, K = x.shape
    N = w.shape[0]
    u8 = dict(dtype=torch.uint8, device="cuda")
    xq, xs = torch.empty((M, K), **u8), torch.empty((M, K // 32), **u8)
    wq, ws = torch.empty((N, K), **u8), torch.empty((N, K // 32), **u8)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step(timer):
        stream = torch.cuda.current_stream().cuda_stream
        _check(timer.run("mx_quant_x", lambda: mx.mx_quantize(
            x.data_ptr(), mx.BF16, M, K, K, mx.E4M3, mx.RULE_FLOOR, xq.data_ptr(), K, xs.data_ptr(), None,
            stream)), "mx")
        _check(timer.run("mx_quant_w", lambda: mx.mx_quantize(
            w.data_ptr(), mx.BF16, N, K, K, mx.E4M3, mx.RULE_FLOOR, wq.data_ptr(), K, ws.data_ptr(), None,
            stream)), "mx")
        _check(timer.run("gemm", lambda: mx.mx_gemm(
            M, N, K, xq.data_ptr(), K, mx.E4M3, xs.data_ptr(), wq.data_ptr(), K, mx.E4M3, ws.data_ptr(),
            y.data_ptr(), N, mx.BF16, stream)), "gemm")

    def cpu(rows):
        import oracle
        th = oracle_threads()
        rows = M if rows <= 0 else min(rows, M)
        t0 = time.perf_counter()
        q, s, _ = oracle.mx_quantize(np.ascontiguousarray(d["x"][:rows]), oracle.E4M3, oracle.RULE_FLOOR, threads=th)
        t1 = time.perf_counter()
        wq_, ws_, _ = oracle.mx_quantize(d["w"], oracle.E4M3, oracle.RULE_FLOOR, threads=th)
        t2 = time.perf_counter()
        oracle.mx_gemm(q, s, oracle.E4M3, wq_, ws_, oracle.E4M3, threads=th)
        t3 = time.perf_counter()
        f = M / float(rows)
        t_step = (t1 - t0) * f + (t2 - t1) + (t3 - t2) * f
        return cpu_line(2.0 * M * N * K / t_step / 1e12, "TFLOP/s", th, t3 - t0,
                        "the full step" if rows == M else "%d of %d rows, scaled" % (rows, M))
    return {"step": step, "outputs": [xq, xs, wq, ws, y],
            "sizes": {"mx_quant_x": M * K * 3 + M * K // 32, "mx_quant_w": N * K * 3 + N * K // 32},
            "flops": 2.0 * M * N * K, "M": M, "N": N, "K": K, "dtype": "fp8_e4m3",
            "gemm_bytes": M * K + N * K + (M + N) * (K // 32) + 2 * M * N,
            "desc": "mxfprop1p5b: MX-quantize X 4096x1536 and W 8960x1536 bf16 (32-element E4M3 blocks, OCP "
                    "floor scales) + MX GEMM M=4096 N=8960 K=1536 bf16 out",
            "cpu": cpu}


def w_f32sfprop1p5b():
    import torch
    import mx_block_scaled_x128_amd as mx
    import synth
    d = synth.fprop1p5b()
    x, w = to_dev(d["x"]), to_dev(d["w"])
    M, K = x.shape
    N = w.shape[0]
    u8 = dict(dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    xq, xs = torch.empty((M, K), **u8), torch.empty((M, K // 128), **f32)
    wq, ws = torch.empty((N, K), **u8), torch.empty(((N + 127) // 128, K // 128), **f32)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step(timer):
        stream = torch.cuda.current_stream().cuda_stream
        _check(timer.run("quant_token_x_f32s", lambda: mx.fp8_quantize_token_f32s(
            x.data_ptr(), mx.BF16, M, K, K, mx.ROW, mx.E4M3, xq.data_ptr(), K, xs.data_ptr(), stream)), "q")
        _check(timer.run("quant_block_w_f32s", lambda: mx.fp8_quantize_block_f32s(
            w.data_ptr(), mx.BF16, N, K, K, mx.E4M3, wq.data_ptr(), K, ws.data_ptr(), stream)), "q")
        _check(timer.run("gemm", lambda: mx.fp8_gemm_f32s(
            M, N, K, xq.data_ptr(), K, mx.E4M3, xs.data_ptr(), wq.data_ptr(), K, mx.E4M3, mx.B_NK,
            ws.data_ptr(), mx.SCALE_BLOCK128, y.data_ptr(), N, mx.BF16, stream)), "gemm")

    def cpu(rows):
        import oracle
        th = oracle_threads()
        rows = M if rows <= 0 else min(rows, M)
        t0 = time.perf_counter()
        q, s = oracle.quantize_rows_f32s(np.ascontiguousarray(d["x"][:rows]), oracle.E4M3, threads=th)
        t1 = time.perf_counter()
        wq_, ws_ = oracle.quantize_block_f32s(d["w"], oracle.E4M3, threads=th)
        t2 = time.perf_counter()
        oracle.gemm_f32s(q, s, oracle.E4M3, wq_, ws_, oracle.E4M3, threads=th)
        t3 = time.perf_counter()
        f = M / float(rows)
        t_step = (t1 - t0) * f + (t2 - t1) + (t3 - t2) * f
        return cpu_line(2.0 * M * N * K / t_step / 1e12, "TFLOP/s", th, t3 - t0,
                        "the full step" if rows == M else "%d of %d rows, scaled" % (rows, M))
    return {"step": step, "outputs": [xq, xs, wq, ws, y],
            "sizes": {"quant_token_x_f32s": M * K * 3 + 4 * M * (K // 128),
                      "quant_block_w_f32s": N * K * 3 + 4 * ((N + 127) // 128) * (K // 128)},
            "flops": 2.0 * M * N * K, "M": M, "N": N, "K": K, "dtype": "fp8_e4m3",
            "gemm_bytes": M * K + N * K + 4 * M * (K // 128) + 4 * (N // 128) * (K // 128) + 2 * M * N,
            "desc": "f32sfprop1p5b: token-quantize X 4096x1536 and block-quantize W 8960x1536 bf16 with fp32 "
                    "scales (amax / 448) + GEMM over fp32-scaled operands M=4096 N=8960 K=1536 bf16 out",
            "cpu": cpu}


def w_dualq():
    import torch
    import mx_block_scaled_x128_amd as mx
    import synth
    hx = synth.wgrad()["x"]
    hw = synth.dgrad7b(rows=16)["w"]
    x, w = to_dev(hx), to_dev(hw)
    T, C = x.shape
    O, I = w.shape
    u8 = dict(dtype=torch.uint8, device="cuda")
    xq, xs = torch.empty((T, C), **u8), torch.empty((T, C // 128), **u8)
    xqt, xst = torch.empty((C, T), **u8), torch.empty((C, T // 128), **u8)
    wq, ws = torch.empty((O, I), **u8), torch.empty(((O + 127) // 128, I // 128), **u8)
    wqt, wst = torch.empty((I, O), **u8), torch.empty((I // 128, (O + 127) // 128), **u8)

    def step(timer):
        stream = torch.cuda.current_stream().cuda_stream
        _check(timer.run("token_dual_x", lambda: mx.fp8_quantize_token_dual(
            x.data_ptr(), mx.BF16, T, C, C, mx.E4M3, xq.data_ptr(), C, xs.data_ptr(), xqt.data_ptr(), T,
            xst.data_ptr(), stream)), "dual")
        _check(timer.run("block_dual_w", lambda: mx.fp8_quantize_block_dual(
            w.data_ptr(), mx.BF16, O, I, I, mx.E4M3, wq.data_ptr(), I, ws.data_ptr(), wqt.data_ptr(), O,
            wst.data_ptr(), stream)), "dual")
    sizes = {"token_dual_x": T * C * 4 + 2 * T * C // 128,
             "block_dual_w": O * I * 4 + 2 * ((O + 127) // 128) * (I // 128)}

    def cpu(rows):
        import oracle
        th = oracle_threads()
        t0 = time.perf_counter()
        oracle.quantize_rows(hx, oracle.E4M3, threads=th)
        oracle.quantize_cols_t(hx, oracle.E4M3, threads=th)
        q, _ = oracle.quantize_block(hw, oracle.E4M3, threads=th)
        np.ascontiguousarray(q.T)
        t1 = time.perf_counter()
        return cpu_line(sum(sizes.values()) / (t1 - t0) / 1e9, "GB/s", th, t1 - t0,
                        "the full step (row and transposed-column codes of X, block codes of W and their "
                        "transpose)")
    return {"step": step, "outputs": [xq, xs, xqt, xst, wq, ws, wqt, wst], "sizes": sizes, "flops": 0.0,
            "M": 0, "N": 0, "K": 0, "dtype": "fp8_e4m3",
            "desc": "dualq: X 16384x4096 bf16 -> 1x128 row codes + 128-token column codes (transposed), one read; "
                    "W 18944x3584 bf16 -> 128x128 block codes + their transpose",
            "cpu": cpu}


def w_gaussws7b():
    import torch
    import mx_block_scaled_x128_amd as mx
    import synth
    wf = synth.bf16_bits_to_f32(synth.dgrad7b(rows=16)["w"]).astype(np.float32)
    R, C = wf.shape
    bt_np = np.random.default_rng(10).integers(4, 9, (-(-R // 32), -(-C // 32))).astype(np.int8)
    w = to_dev(wf)
    bt = torch.from_numpy(bt_np).cuda()
    w_hat = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")

    def step(timer):
        stream = torch.cuda.current_stream().cuda_stream
        _check(timer.run("gaussws", lambda: mx.gaussws_sample(
            w.data_ptr(), mx.F32, R, C, C, bt.data_ptr(), 2025, 7, w_hat.data_ptr(), C, stream)), "gws")
    sizes = {"gaussws": R * C * 6 + bt_np.size}

    def cpu(rows):
        import oracle
        th = oracle_threads()
        t0 = time.perf_counter()
        oracle.gaussws(wf, bt_np, 2025, 7, threads=th)
        t1 = time.perf_counter()
        return cpu_line(sizes["gaussws"] / (t1 - t0) / 1e9, "GB/s", th, t1 - t0, "the full step")
    return {"step": step, "outputs": [w_hat], "sizes": sizes, "flops": 0.0, "M": 0, "N": 0, "K": 0,
            "dtype": "bf16",
            "desc": "gaussws7b: GaussWS sampled weight of W 18944x3584 fp32 master weights (32x32 blocks, int8 "
                    "bitwidths 4..8, Philox4x64-10 rounded-normal noise) -> bf16",
            "cpu": cpu}


E4M3_TOP = 0x7E


def mx_clamp_stats(q, cnt, clustered_rows):
    """Clamp statistics of one tensor's MX codes and counts (numpy), split into the
    clustered rows [0, clustered_rows) and the others: per block, the fraction of its
    32 values whose scaled magnitude exceeded the largest code (strict clamp); the
    fraction of values on the top code; the fraction of blocks whose 32 codes are all
    one code."""
    out = {}
    for part, sl in (("clustered", slice(0, clustered_rows)), ("normal", slice(clustered_rows, None))):
        c = cnt[sl].astype(np.int64)
        qq = q[sl]
        blocks = qq.reshape(qq.shape[0], -1, 32)
        out[part] = {
            "values": int(qq.size), "blocks": int(c.size), "clamped": int(c.sum()),
            "blocks_with_clamp": int((c > 0).sum()), "max_clamped_in_block": int(c.max()),
            "top_code": int(((qq & 0x7F) == E4M3_TOP).sum()),
            "single_code_blocks": int((blocks == blocks[:, :, :1]).all(axis=2).sum())}
    return out


def w_mxstress():
    import torch
    import mx_block_scaled_x128_amd as mx
    import synth
    ntens = 64
    hosts = [synth.mxstress_tensor(j) for j in range(ntens)]
    xs_ = [to_dev(h) for h in hosts]
    R, C = xs_[0].shape
    u8 = dict(dtype=torch.uint8, device="cuda")
    q, sc, cn = torch.empty((R, C), **u8), torch.empty((R, C // 32), **u8), torch.empty((R, C // 32), **u8)

    def step(timer):
        stream = torch.cuda.current_stream().cuda_stream
        for st in timer.run_many("mx_quant", [lambda j=j: mx.mx_quantize(
                xs_[j].data_ptr(), mx.F32, R, C, C, mx.E4M3, mx.RULE_FLOOR, q.data_ptr(), C, sc.data_ptr(),
                cn.data_ptr(), stream) for j in range(ntens)]):
            _check(st, "mx")
    sizes = {"mx_quant": R * C * 5 + 2 * R * (C // 32)}

    def device_stats():
        """Clamp statistics of every tensor from the device's codes and counts."""
        per = []
        for j in range(ntens):
            qd, _, cd = mx.quantize_mx(xs_[j], mx.E4M3, mx.RULE_FLOOR, counts=True)
            per.append(mx_clamp_stats(qd.cpu().numpy(), cd.cpu().numpy(), R // 2))
        return per

    def cpu(rows):
        import oracle
        th = oracle_threads()
        t0 = time.perf_counter()
        ref = []
        for h in hosts:
            qr, _, cr = oracle.mx_quantize(h, oracle.E4M3, oracle.RULE_FLOOR, threads=th)
            ref.append((qr, cr))
        t1 = time.perf_counter()
        line = cpu_line(sizes["mx_quant"] * ntens / (t1 - t0) / 1e9, "GB/s", th, t1 - t0,
                        "all 64 tensors (the full step)")
        return line, [mx_clamp_stats(qr, cr, R // 2) for qr, cr in ref]
    return {"step": step, "outputs": [q, sc, cn], "sizes": sizes, "flops": 0.0, "M": 0, "N": 0, "K": 0,
            "dtype": "fp8_e4m3", "calls": {"mx_quant": ntens}, "device_stats": device_stats,
            "desc": "mxstress: 64 tensors 4096x4096 fp32 (rows [0,2048) 1 + N(0,1e-3), rows [2048,4096) N(0,1)), "
                    "MX 32-element E4M3 blocks, OCP floor scales, clamp counts",
            "cpu": cpu}


def summarize_stats(per):
    """Totals over tensors, as fractions: values clamped, blocks with a clamp, the
    largest per-block clamped fraction, values on the top code, single-code blocks."""
    out = {}
    for part in ("normal", "clustered"):
        tot = {k: sum(p[part][k] for p in per) for k in ("values", "blocks", "clamped", "blocks_with_clamp",
                                                        "top_code", "single_code_blocks")}
        out[part] = {
            "clamped_fraction": tot["clamped"] / tot["values"],
            "mean_clamped_fraction_per_block": tot["clamped"] / (32.0 * tot["blocks"]),
            "max_clamped_fraction_in_a_block": max(p[part]["max_clamped_in_block"] for p in per) / 32.0,
            "blocks_with_a_clamp": tot["blocks_with_clamp"] / tot["blocks"],
            "top_code_fraction": tot["top_code"] / tot["values"],
            "single_code_block_fraction": tot["single_code_blocks"] / tot["blocks"],
            "counts": tot}
    return out


SETUP = {"dgrad7b": w_dgrad7b, "fprop1p5b": w_fprop1p5b, "wgrad": w_wgrad, "mxfprop1p5b": w_mxfprop1p5b,
         "f32sfprop1p5b": w_f32sfprop1p5b, "dualq": w_dualq, "gaussws7b": w_gaussws7b, "mxstress": w_mxstress}


def bench_workload(args):
    wl = SETUP[args.workload]()
    step, sizes, flops = wl["step"], wl["sizes"], wl["flops"]
    calls = wl.get("calls", {})
    ramp_steps = ramp(step, min_steps=args.warmup)
    per_step = time_plain(step, args.steps, args.warmup)
    per_step_events, timer = time_steps(step, args.steps, args.warmup)
    per_step_graph, per_graph = time_graph(step, args.steps, args.warmup, wl["outputs"])
    kern = {}
    for name, b in sizes.items():
        t = timer.mean(name)
        kern[name] = {"us": round(t * 1e6, 2), "GB/s": round(b / t / 1e9, 1),
                      "frac_hbm_peak": round(b / t / 1e9 / HBM_PEAK_GBS, 4), "bytes": b}
    traffic = recorded_traffic(args.workload)
    if flops:
        g = timer.mean("gemm")
        gb = back_to_back(step, "gemm", max(20, args.steps))
        kern["gemm"] = {"us": round(g * 1e6, 2), "TFLOP/s": round(flops / g / 1e12, 1),
                        "frac_fp8_peak": round(flops / g / 1e12 / FP8_PEAK_TFLOPS, 4), "flops": flops,
                        "us_back_to_back": round(gb * 1e6, 2)}
        value, unit = flops / per_step / 1e12, "TFLOP/s"
        roof = {"bound": "mfma", "achieved": round(flops / g / 1e12, 2), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(flops / g / 1e12 / FP8_PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel": "gemm",
                "traffic_note": "HBM bytes per GEMM call (FETCH_SIZE + WRITE_SIZE, copy-calibrated; "
                                "profiles/traffic_%s.json); algorithmic bytes %d" % (args.workload, wl["gemm_bytes"])}
    else:
        tot = sum(b * calls.get(name, 1) for name, b in sizes.items())
        value, unit = tot / per_step / 1e9, "GB/s"
        dom = max(sizes, key=lambda k: kern[k]["us"])
        roof = {"bound": "hbm", "achieved": kern[dom]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": kern[dom]["frac_hbm_peak"], "traffic": traffic, "kernel": dom,
                "traffic_note": "HBM bytes per call of %s (FETCH_SIZE + WRITE_SIZE, copy-calibrated; "
                                "profiles/traffic_%s.json); algorithmic bytes %d" % (dom, args.workload, sizes[dom])}
    config = {"workload": wl["desc"]}
    if flops:
        config.update({"M": wl["M"], "N": wl["N"], "K": wl["K"]})
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(per_step * 1e3, 4),
        "ms_per_step_with_events": round(per_step_events * 1e3, 4),
        "ms_per_step_graph": round(per_step_graph * 1e3, 4), "steps_per_graph": per_graph,
        "clock_ramp_steps": ramp_steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl["dtype"],
        "data": "synthetic (seeded numpy PCG64; inputs resident in HBM before timing)",
        "config": config, "kernels": kern, "roofline": roof,
    }
    if args.workload != "mxstress":  # 64 launches per step: the scrubbed pass would take long
        per, device = context_measurements(step, timer)
        for name, d in per.items():
            if name in line["kernels"]:
                line["kernels"][name].update(d)
        line["device"] = device
    line["timing"] = ("before any timing, clock_ramp_steps untimed steps (at least 0.3 s of sustained load, at "
                      "least `warmup`) bring the GPU clock to its loaded steady state; then `warmup` untimed "
                      "steps before each timed pass. "
                      "value: `steps` whole steps launched back to back between two device synchronisations "
                      "(ms_per_step); kernels.us: mean of event-bracketed calls in a second pass of `steps` steps "
                      "(ms_per_step_with_events), on the stream they run on (mxstress: one event pair around a step's 64 "
                      "launches, divided by 64) "
                      "(us_median: median); us_cold_median: each call after a 512 MiB scrub read (no input in "
                      "the caches, which hold clean lines), us_cold_dirty_median: after a 512 MiB scrub write "
                      "(the caches' dirty lines are written back during the call), medians of 10; "
                      "roofline.achieved: from kernels.<kernel>.us; gemm.us_back_to_back: mean of GEMM calls "
                      "issued back to back between one event pair (operands left in the caches by the previous "
                      "call: context, not the step); ms_per_step_graph: replays of a HIP graph of steps_per_graph "
                      "steps (context: the captured step reproduces the eager outputs bit for bit)")
    cpu_stats = None
    if args.no_cpu:
        line["cpu_baseline"] = None
    elif args.workload == "mxstress":
        line["cpu_baseline"], cpu_stats = wl["cpu"](args.cpu_rows)
    else:
        line["cpu_baseline"] = wl["cpu"](args.cpu_rows)
    if "device_stats" in wl:
        per = wl["device_stats"]()
        line["clamp_stats"] = summarize_stats(per)
        line["clamp_stats"]["oracle_check"] = (
            "not run (--no-cpu)" if cpu_stats is None else
            "the oracle's codes and counts give the same statistics for %d of %d tensors"
            % (sum(a == b for a, b in zip(per, cpu_stats)), len(per)))
    return line


def bench_gemm_sweep(args):
    """The block-scaled GEMM at M = 4096 over N and K, bf16 output (and fp32 output at one
    shape), uniformly random finite E4M3 codes with scale bytes in [120, 134]: one round of
    256x256 tiles at N = 4096 (256 tiles, one per CU), two rounds at N = 8192; at N = 2048
    the 512 tiles of 128x128 (two workgroups per CU), at N = 2560 one partial round of 160
    256x256 tiles (the two sides of the tile-size choice).  Per shape,
    `warmup` calls and then `steps` calls back to back between one event pair (mean per
    call).  A least-squares line through the one-round bf16 points, time = fixed + slope x
    (K / 128), separates the cost of a round that does not scale with K (prologue, output
    write) from the K loop."""
    import torch
    import mx_block_scaled_x128_amd as mx
    import synth
    M = 4096
    shapes = [(4096, 256, True), (4096, 512, True), (4096, 1536, True), (4096, 3072, True), (4096, 6144, True),
              (8192, 1536, True), (4096, 1536, False), (2048, 4096, True), (2048, 8192, True), (2560, 4096, True)]
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
            "config": {"workload": "gemmsweep: M=4096, N in {2048, 2560, 4096, 8192}, K in {256 .. 8192}"},
            "sweep": res, "fit_one_round_bf16": {"fixed_us": round(float(fixed), 2),
                                                 "us_per_k_block": round(float(slope), 3)},
            "roofline": {"bound": "mfma", "achieved": best["TFLOP/s"], "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(best["TFLOP/s"] / FP8_PEAK_TFLOPS, 4), "traffic": None},
            "cpu_baseline": None}


def bench_vendor_gemm(args):
    """This library's GEMMs beside the ROCm BLAS library's FP8 products (torch._scaled_mm,
    which dispatches to hipBLASLt) on the dgrad7b, fprop1p5b and wgrad shapes: per-tensor
    scales (the least work: one scale for each operand), per-row/per-column scales, and
    32-element E8M0 (MX) scales, against this library's 128x128-block and MX GEMMs.  Both
    sides read the same E4M3 codes (a bf16 N(0, 1/4) draw cast to E4M3, B stored [N][K])
    with unit scales, so every variant computes the same product; bf16 output.  Each
    variant is timed over `steps` calls back to back between one event pair, in three
    interleaved rounds (the median is kept), after a clock ramp.  A variant that the
    library rejects is reported with its error text."""
    import torch
    import mx_block_scaled_x128_amd as mx
    shapes = [("dgrad7b", 8192, 3584, 18944), ("fprop1p5b", 4096, 8960, 1536), ("wgrad", 4096, 4096, 16384)]
    gen = torch.Generator(device="cuda").manual_seed(11)
    res = []
    for name, M, N, K in shapes:
        a = (torch.randn(M, K, device="cuda", generator=gen) * 0.5).to(torch.float8_e4m3fn)
        bt = (torch.randn(N, K, device="cuda", generator=gen) * 0.5).to(torch.float8_e4m3fn)
        au, bu = a.view(torch.uint8), bt.view(torch.uint8)
        one = torch.ones((), device="cuda")
        rows, cols = torch.ones(M, 1, device="cuda"), torch.ones(1, N, device="cuda")
        mxa = torch.full((M, K // 32), 127, dtype=torch.uint8, device="cuda")
        mxb = torch.full((N, K // 32), 127, dtype=torch.uint8, device="cuda")
        sa = torch.full((M, K // 128), 127, dtype=torch.uint8, device="cuda")
        sb = torch.full(((N + 127) // 128, K // 128), 127, dtype=torch.uint8, device="cuda")
        out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        variants = {
            "this: 128x128-block scales": lambda: mx.block_scaled_gemm(au, sa, mx.E4M3, bu, sb, mx.E4M3, mx.B_NK,
                                                                       mx.SCALE_BLOCK128, out=out),
            "this: MX scales": lambda: mx.mx_scaled_gemm(au, mxa, mx.E4M3, bu, mxb, mx.E4M3, out=out),
            "hipBLASLt: per-tensor scales": lambda: torch._scaled_mm(a, bt.t(), scale_a=one, scale_b=one,
                                                                     out_dtype=torch.bfloat16),
            "hipBLASLt: per-row/column scales": lambda: torch._scaled_mm(a, bt.t(), scale_a=rows, scale_b=cols,
                                                                         out_dtype=torch.bfloat16),
            "hipBLASLt: MX scales": lambda: torch._scaled_mm(a, bt.t(), scale_a=mxa.view(torch.float8_e8m0fnu),
                                                             scale_b=mxb.view(torch.float8_e8m0fnu),
                                                             out_dtype=torch.bfloat16),
        }
        errors, times = {}, {k: [] for k in variants}
        ref = None
        for k, f in list(variants.items()):
            try:
                y = f()
                torch.cuda.synchronize()
                y = out if y is None else y
                if ref is None:
                    ref = y.float().clone()
                elif not torch.allclose(y.float(), ref, rtol=2 ** -7, atol=1e-2 * float(ref.abs().max())):
                    errors[k] = "output differs from this library's block-scaled product"
            except Exception as e:  # a scaling mode the installed library does not offer
                errors[k] = str(e).splitlines()[0][:160]
                del variants[k]
        ramp(lambda timer: variants["this: 128x128-block scales"](), 0.3)
        for _ in range(3):
            for k, f in variants.items():
                for _ in range(args.warmup):
                    f()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(args.steps):
                    f()
                e1.record()
                torch.cuda.synchronize()
                times[k].append(e0.elapsed_time(e1) * 1e3 / args.steps)
        for k in times:
            if times[k]:
                us = float(np.median(times[k]))
                res.append({"shape": name, "M": M, "N": N, "K": K, "gemm": k, "us": round(us, 2),
                            "TFLOP/s": round(2.0 * M * N * K / us / 1e6, 1)})
            if k in errors:
                res.append({"shape": name, "M": M, "N": N, "K": K, "gemm": k, "error": errors[k]})
        del a, bt, au, bu, mxa, mxb, sa, sb, out, ref, variants
    main_line = [r for r in res if r["shape"] == "dgrad7b" and r["gemm"] == "this: 128x128-block scales"][0]
    return {"metric": "FP8 GEMM TFLOP/s beside the ROCm BLAS library's FP8 products", "value": main_line["TFLOP/s"],
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(main_line["us"] / 1e3, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic (bf16 N(0, 1/4) cast to E4M3, unit scales)",
            "config": {"workload": "vendorgemm: dgrad7b 8192x3584x18944, fprop1p5b 4096x8960x1536, "
                                   "wgrad 4096x4096x16384"},
            "comparison": res,
            "roofline": {"bound": "mfma", "achieved": main_line["TFLOP/s"], "peak": FP8_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(main_line["TFLOP/s"] / FP8_PEAK_TFLOPS, 4), "traffic": None},
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
    if args.workload == "copy":
        line = bench_copy(args)
    elif args.workload == "gemmsweep":
        line = bench_gemm_sweep(args)
    elif args.workload == "vendorgemm":
        line = bench_vendor_gemm(args)
    else:
        line = bench_workload(args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
