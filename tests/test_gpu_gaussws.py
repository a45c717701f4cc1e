"""GPU parity of the GaussWS sampler against the CPU oracle: the sampled
bf16 weights must be bit-identical (the noise is a deterministic function of
(seed, stream, row, col) through Philox4x64-10).  Calls go through the C ABI."""
import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import oracle
import synth
from gpu_helpers import ORACLE_THREADS, dev, dev_ld16, host

pytestmark = pytest.mark.gpu


def bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bitwidths(seed, rows, cols, lo=2, hi=12):
    return np.random.default_rng(seed).integers(lo, hi + 1, (-(-rows // 32), -(-cols // 32))).astype(np.int8)


@pytest.mark.parametrize("bf16_in", [False, True])
@pytest.mark.parametrize("shape", [(1, 8), (37, 200), (64, 256), (130, 520), (300, 1024 + 8)])
def test_parity(bf16_in, shape):
    rows, cols = shape
    w = synth.weights_like(rows * 5 + cols, shape, bf16=bf16_in)
    bt = bitwidths(rows + cols, rows, cols)
    seed, stream_id = 0x1234_5678_9ABC_DEF0 + rows, cols
    out = mx.gaussws(dev_ld16(w), torch.from_numpy(bt).cuda(), seed, stream_id)
    torch.cuda.synchronize()
    ref = oracle.gaussws(w, bt, seed, stream_id)
    assert np.array_equal(bits(out), ref)


def test_extreme_bitwidths_and_tiny_blocks():
    """Blocks of fp32 subnormals (subnormal noise steps), very large and very
    small bitwidths (noise steps that overflow to inf or underflow to zero)."""
    rows, cols = 64, 128
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((rows, cols)) * 0.5).astype(np.float32)
    w[:32, :32] = (rng.standard_normal((32, 32)) * 1e-39).astype(np.float32)
    w[32:, :32] = (rng.standard_normal((32, 32)) * 3e38 / 5).astype(np.float32)
    bt = np.array([[12, 127, -100, 1], [-120, 24, 0, -1]], np.int8)
    out = mx.gaussws(dev(w), torch.from_numpy(bt).cuda(), 77, 5)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), oracle.gaussws(w, bt, 77, 5))


def test_leading_dimensions_and_padding():
    rows, cols = 96, 200
    w = synth.weights_like(6, (rows, cols), bf16=False)
    bt = bitwidths(7, rows, cols)
    wd = dev(w, pitch=224)
    out = torch.full((rows, 256), -7.0, dtype=torch.bfloat16, device="cuda")
    btd = torch.from_numpy(bt).cuda()
    st = mx.gaussws_sample(wd.data_ptr(), mx.F32, rows, cols, 224, btd.data_ptr(), 5, 6, out.data_ptr(), 256,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    ob = bits(out)
    assert np.array_equal(ob[:, :cols], oracle.gaussws(w, bt, 5, 6))
    assert np.all(host(out)[:, cols:] == -7.0)


def test_deterministic_and_stream_dependent():
    w = dev(synth.weights_like(8, (128, 256), bf16=True))
    bt = torch.from_numpy(bitwidths(9, 128, 256)).cuda()
    a = bits(mx.gaussws(w, bt, 42, 0))
    b = bits(mx.gaussws(w, bt, 42, 0))
    c = bits(mx.gaussws(w, bt, 42, 1))
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_dgrad_weight_full_size():
    """W 18944 x 3584 (the 7B-class layer's weight), fp32 master weights,
    bitwidths 4..8: the whole sampled tensor compared bit for bit."""
    w = synth.bf16_bits_to_f32(synth.dgrad7b(rows=16)["w"]).astype(np.float32)
    rows, cols = w.shape
    bt = bitwidths(10, rows, cols, 4, 8)
    out = mx.gaussws(dev(w), torch.from_numpy(bt).cuda(), 2025, 7)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), oracle.gaussws(w, bt, 2025, 7, threads=ORACLE_THREADS))


def test_tall_input_beyond_65535_strip_rows():
    """More than 65535 strips of 32 rows: the sampler runs on a 1-D grid."""
    rows, cols = 65536 * 32 + 32, 8
    w = synth.weights_like(124, (rows, cols), bf16=False)
    bt = bitwidths(125, rows, cols)
    out = mx.gaussws(dev_ld16(w), torch.from_numpy(bt).cuda(), 3, 4)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), oracle.gaussws(w, bt, 3, 4, threads=ORACLE_THREADS))
