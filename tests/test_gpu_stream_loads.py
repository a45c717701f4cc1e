"""The quantizers and the sampler read inputs of 64 MiB or more with
non-temporal loads and smaller ones with ordinary loads: the same arithmetic
behind a different cache policy.  A 64 MiB input and its leading 256 rows (a
2 MiB input, read the other way) must give the same codes, scales and sampled
weights bit for bit on those rows.  (The full-size workload tests compare the
streaming path with the oracle for the E8M0 quantizers and the sampler; this
covers the fp32-scale quantizers' streaming path too.)  Calls go through the
C ABI."""
import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import synth
from gpu_helpers import dev

pytestmark = pytest.mark.gpu

ROWS, COLS, HEAD = 8192, 4096, 256   # bf16: 64 MiB; the head: 2 MiB


@pytest.fixture(scope="module")
def x_bf16():
    x = dev(synth.heavy_tail_like(5150, (ROWS, COLS), bf16=True))
    assert x.numel() * x.element_size() == 64 << 20
    return x


def same(a, b):
    assert a.dtype == b.dtype and a.shape == b.shape
    assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float32 else a,
                       b.view(torch.uint8) if b.dtype == torch.float32 else b)


@pytest.mark.parametrize("fmt", [mx.E4M3, mx.E5M2])
@pytest.mark.parametrize("f32s", [False, True])
def test_token_rows(x_bf16, fmt, f32s):
    fn = mx.quantize_token_f32s if f32s else mx.quantize_token
    q, s = fn(x_bf16, fmt, mx.ROW)
    qh, sh = fn(x_bf16[:HEAD], fmt, mx.ROW)
    torch.cuda.synchronize()
    same(qh, q[:HEAD])
    same(sh, s[:HEAD])


@pytest.mark.parametrize("fmt", [mx.E4M3, mx.E5M2])
@pytest.mark.parametrize("f32s", [False, True])
def test_token_cols_t(x_bf16, fmt, f32s):
    fn = mx.quantize_token_f32s if f32s else mx.quantize_token
    qt, st = fn(x_bf16, fmt, mx.COL_T)
    qth, sth = fn(x_bf16[:HEAD], fmt, mx.COL_T)
    torch.cuda.synchronize()
    same(qth, qt[:, :HEAD])
    same(sth, st[:, :HEAD // 128])


@pytest.mark.parametrize("fmt", [mx.E4M3, mx.E5M2])
@pytest.mark.parametrize("f32s", [False, True])
def test_block(x_bf16, fmt, f32s):
    fn = mx.quantize_block_f32s if f32s else mx.quantize_block
    q, s = fn(x_bf16, fmt)
    qh, sh = fn(x_bf16[:HEAD], fmt)
    torch.cuda.synchronize()
    same(qh, q[:HEAD])
    same(sh, s[:HEAD // 128])


@pytest.mark.parametrize("fmt", [mx.E4M3, mx.E5M2])
def test_token_dual(x_bf16, fmt):
    q, s, qt, st = mx.quantize_token_dual(x_bf16, fmt)
    qh, sh, qth, sth = mx.quantize_token_dual(x_bf16[:HEAD], fmt)
    torch.cuda.synchronize()
    same(qh, q[:HEAD])
    same(sh, s[:HEAD])
    same(qth, qt[:, :HEAD])
    same(sth, st[:, :HEAD // 128])


@pytest.mark.parametrize("fmt", [mx.E4M3, mx.E5M2])
def test_block_dual(x_bf16, fmt):
    q, s, qt, st = mx.quantize_block_dual(x_bf16, fmt)
    qh, sh, qth, sth = mx.quantize_block_dual(x_bf16[:HEAD], fmt)
    torch.cuda.synchronize()
    same(qh, q[:HEAD])
    same(sh, s[:HEAD // 128])
    same(qth, qt[:, :HEAD])
    same(sth, st[:, :HEAD // 128])


def test_gaussws_fp32():
    w = dev(synth.weights_like(5151, (4096, 4096), bf16=False))   # fp32: 64 MiB
    assert w.numel() * w.element_size() == 64 << 20
    bt = torch.from_numpy(np.random.default_rng(5152).integers(2, 9, size=(128, 128)).astype(np.int8)).cuda()
    out = mx.gaussws(w, bt, 909, 3)
    outh = mx.gaussws(w[:HEAD], bt[:HEAD // 32].contiguous(), 909, 3)
    torch.cuda.synchronize()
    same(outh, out[:HEAD])
