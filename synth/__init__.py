"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module draws random tensors and nothing else: it holds none of the
quantization or GEMM arithmetic.  Every draw uses numpy's PCG64
(``numpy.random.default_rng(seed)``) in fp64; fp32 tensors are the fp64 draws
cast with round-to-nearest-even, bf16 tensors are those fp32 values cast to
bf16 by torch (round-to-nearest-even) and returned as raw uint16 patterns.

Workloads (shapes and distributions of the FP8 training pages' linear layers;
"N(0, s)" means standard deviation s, "Laplace(0, b)" scale b):
  tiny       X 256x512 fp32 N(0,1), 0.5% of entries x100; W 256x512 fp32 N(0,0.02); seed 0
  fprop1p5b  X 4096x1536 bf16 N(0,1) times a per-channel factor exp(U(ln 0.1, ln 30));
             W 8960x1536 bf16 N(0,0.02); seeds 1000, 1001
  dgrad7b    dY 8192x18944 bf16 Laplace(0,1e-3); W 18944x3584 bf16 N(0,0.015); seeds 2000, 2001
  mxstress   64 tensors 4096x4096 fp32: rows [0,2048) 1 + N(0,1e-3), rows [2048,4096) N(0,1);
             seed 3000 + j for tensor j
  wgrad      X 16384x4096 bf16 Student-t(3) x 0.5; dY 16384x4096 bf16 N(0,1e-4); seeds 4000, 4001
The ``*_like`` helpers draw the same distributions at other (small, ragged)
shapes for parity tests.
"""
import numpy as np

_TORCH = None


def _torch():
    global _TORCH
    if _TORCH is None:
        import torch
        _TORCH = torch
    return _TORCH


def to_f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def to_bf16_bits(a):
    """fp64/fp32 array -> bf16 bit patterns (uint16), round-to-nearest-even via torch."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to fp32 (for reporting and checks)."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ distributions

def outlier_normal(rng, shape, frac=0.005, factor=100.0):
    x = rng.standard_normal(shape)
    mask = rng.random(shape) < frac
    x[mask] *= factor
    return x


def channel_scaled_normal(rng, shape, lo=0.1, hi=30.0):
    x = rng.standard_normal(shape)
    s = np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape[1]))
    return x * s[None, :]


def clustered_or_normal(rng, shape, sd=1e-3):
    """First half of the rows 1 + N(0, sd) (layer-norm-like), second half N(0,1)."""
    rows = shape[0]
    h = rows // 2
    x = np.empty(shape)
    x[:h] = 1.0 + rng.normal(0.0, sd, size=(h,) + tuple(shape[1:]))
    x[h:] = rng.standard_normal((rows - h,) + tuple(shape[1:]))
    return x


# ---------------------------------------------------------------------- workloads

def tiny():
    rng = np.random.default_rng(0)
    x = to_f32(outlier_normal(rng, (256, 512)))
    w = to_f32(rng.normal(0.0, 0.02, size=(256, 512)))
    return {"x": x, "w": w}


def fprop1p5b(rows=4096):
    x = to_bf16_bits(channel_scaled_normal(np.random.default_rng(1000), (rows, 1536)))
    w = to_bf16_bits(np.random.default_rng(1001).normal(0.0, 0.02, size=(8960, 1536)))
    return {"x": x, "w": w}


def dgrad7b(rows=8192):
    dy = to_bf16_bits(np.random.default_rng(2000).laplace(0.0, 1e-3, size=(rows, 18944)))
    w = to_bf16_bits(np.random.default_rng(2001).normal(0.0, 0.015, size=(18944, 3584)))
    return {"dy": dy, "w": w}


def mxstress_tensor(j, rows=4096, cols=4096):
    return to_f32(clustered_or_normal(np.random.default_rng(3000 + j), (rows, cols)))


def wgrad(tokens=16384, channels=4096):
    x = to_bf16_bits(np.random.default_rng(4000).standard_t(3, size=(tokens, channels)) * 0.5)
    dy = to_bf16_bits(np.random.default_rng(4001).normal(0.0, 1e-4, size=(tokens, channels)))
    return {"x": x, "dy": dy}


# ------------------------------------------------------------ small-shape variants

def activations_like(seed, shape, bf16=True):
    x = channel_scaled_normal(np.random.default_rng(seed), shape)
    return to_bf16_bits(x) if bf16 else to_f32(x)


def outliers_like(seed, shape, bf16=False):
    x = outlier_normal(np.random.default_rng(seed), shape)
    return to_bf16_bits(x) if bf16 else to_f32(x)


def weights_like(seed, shape, sd=0.02, bf16=True):
    x = np.random.default_rng(seed).normal(0.0, sd, size=shape)
    return to_bf16_bits(x) if bf16 else to_f32(x)


def gradients_like(seed, shape, b=1e-3, bf16=True):
    x = np.random.default_rng(seed).laplace(0.0, b, size=shape)
    return to_bf16_bits(x) if bf16 else to_f32(x)


def heavy_tail_like(seed, shape, bf16=True):
    x = np.random.default_rng(seed).standard_t(3, size=shape) * 0.5
    return to_bf16_bits(x) if bf16 else to_f32(x)


def mx_like(seed, shape):
    return to_f32(clustered_or_normal(np.random.default_rng(seed), shape))


def random_codes(seed, shape, fmt):
    """Uniformly random finite FP8 codes (NaN and inf patterns redrawn as 0)."""
    c = np.random.default_rng(seed).integers(0, 256, size=shape, dtype=np.uint8)
    if fmt == 0:
        bad = (c & 0x7F) == 0x7F
    else:
        bad = (c & 0x7C) == 0x7C
    c[bad] = 0
    return c


def random_scale_bytes(seed, shape, lo=120, hi=134):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape, dtype=np.uint8)
