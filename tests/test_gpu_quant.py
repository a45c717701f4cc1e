"""GPU parity of the quantizers against the CPU oracle: codes and scale bytes
(and MX clamp counts) must be bit-identical.  Calls go through the C ABI."""
import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import oracle
import synth
from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu

FMTS = [(mx.E4M3, oracle.E4M3), (mx.E5M2, oracle.E5M2)]


def edge_case_rows(bf16):
    """Rows whose groups hit the degenerate cases: all zeros, signed zeros, subnormal inputs,
    exact powers of two, amax at fmax * 2^k and just above, huge and tiny magnitudes, ties."""
    rng = np.random.default_rng(99)
    rows = []
    rows.append(np.zeros(256))
    rows.append(np.array([-0.0] * 128 + [0.0] * 128))
    sub = np.float32(1e-40)  # fp32 subnormal
    rows.append(np.concatenate([np.full(128, sub) * rng.integers(-3, 4, 128), rng.standard_normal(128) * 1e-38]))
    rows.append(np.concatenate([2.0 ** np.arange(-64, 64), -(2.0 ** np.arange(-64, 64))]))
    rows.append(np.concatenate([np.full(128, 448.0 * 2 ** -5), np.full(128, 448.0 * 2 ** -5 * (1 + 2 ** -20))]))
    rows.append(np.concatenate([np.full(128, 57344.0 * 2 ** 3), rng.standard_normal(128) * 3e38 / 4]))
    rows.append(np.concatenate([rng.standard_normal(128) * 1e-30, rng.standard_normal(128) * 1e30]))
    ties = np.array([464.0, 432.0, 400.0, 2.875 * 128, 2.625 * 128, 1.0 / 1024, 3.0 / 1024, 448.0])
    rows.append(np.concatenate([np.tile(ties, 16), -np.tile(ties, 16)]))
    x = np.stack(rows).astype(np.float32)
    return synth.to_bf16_bits(x) if bf16 else x


SHAPES = [(1, 16), (3, 128), (37, 3 * 128 + 48), (256, 512), (130, 1024 + 16)]


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_token_rows_parity(fmt, ofmt, bf16, shape):
    x = synth.outliers_like(shape[0] * 7 + shape[1], shape, bf16=bf16)
    q, s = mx.quantize_token(dev(x), fmt, mx.ROW)
    q_ref, s_ref = oracle.quantize_rows(x, ofmt)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(s), s_ref)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("bf16", [False, True])
def test_token_rows_edge_cases(fmt, ofmt, bf16):
    x = edge_case_rows(bf16)
    q, s = mx.quantize_token(dev(x), fmt, mx.ROW)
    q_ref, s_ref = oracle.quantize_rows(x, ofmt)
    torch.cuda.synchronize()
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(q), q_ref)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_token_rows_leading_dimensions(fmt, ofmt):
    x = synth.activations_like(5, (50, 384), bf16=True)
    xd = dev(x, pitch=400)  # ldx > cols
    q = torch.full((50, 512), 0xCD, dtype=torch.uint8, device="cuda")
    s = torch.empty((50, 3), dtype=torch.uint8, device="cuda")
    st = mx.fp8_quantize_token(xd.data_ptr(), mx.BF16, 50, 384, 400, mx.ROW, fmt, q.data_ptr(), 512,
                               s.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    q_ref, s_ref = oracle.quantize_rows(x, ofmt)
    torch.cuda.synchronize()
    qh = host(q)
    assert np.array_equal(qh[:, :384], q_ref)
    assert np.all(qh[:, 384:] == 0xCD)  # bytes beyond the row untouched
    assert np.array_equal(host(s), s_ref)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shape", [(16, 16), (48, 128), (3 * 128 + 16, 2 * 128 + 48), (512, 256)])
def test_token_cols_t_parity(fmt, ofmt, bf16, shape):
    x = synth.heavy_tail_like(shape[0] + 3 * shape[1], shape, bf16=bf16)
    qt, st = mx.quantize_token(dev(x), fmt, mx.COL_T)
    qt_ref, st_ref = oracle.quantize_cols_t(x, ofmt)
    torch.cuda.synchronize()
    assert np.array_equal(host(qt), qt_ref)
    assert np.array_equal(host(st), st_ref)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_token_cols_t_edge_cases(fmt, ofmt):
    x = np.ascontiguousarray(edge_case_rows(False).T)  # 256 tokens x 8 channels -> pad to 16 channels
    x = np.concatenate([x, x[:, ::-1] * np.float32(0.5)], axis=1).astype(np.float32)
    qt, st = mx.quantize_token(dev(x), fmt, mx.COL_T)
    qt_ref, st_ref = oracle.quantize_cols_t(x, ofmt)
    torch.cuda.synchronize()
    assert np.array_equal(host(st), st_ref)
    assert np.array_equal(host(qt), qt_ref)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shape", [(1, 16), (128, 128), (128 + 40, 2 * 128 + 16), (300, 512)])
def test_block_parity(fmt, ofmt, bf16, shape):
    w = synth.weights_like(shape[0] * 3 + shape[1], shape, bf16=bf16)
    w_np = w
    q, s = mx.quantize_block(dev(w_np), fmt)
    q_ref, s_ref = oracle.quantize_block(w_np, ofmt)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(s), s_ref)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_block_edge_cases(fmt, ofmt):
    x = edge_case_rows(False)
    w = np.zeros((256, 256), np.float32)
    w[:8] = x
    w[130:138] = x[::-1]
    w[200, 3] = 1e-41
    q, s = mx.quantize_block(dev(w), fmt)
    q_ref, s_ref = oracle.quantize_block(w, ofmt)
    torch.cuda.synchronize()
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(q), q_ref)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("rule", [mx.RULE_FLOOR, mx.RULE_CEIL])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shape", [(1, 32), (5, 96), (64, 512 + 32), (257, 1024)])
def test_mx_parity(fmt, ofmt, rule, bf16, shape):
    x = synth.mx_like(shape[0] + 11 * shape[1], shape)
    if bf16:
        x = synth.to_bf16_bits(x)
    q, s, c = mx.quantize_mx(dev(x), fmt, rule, counts=True)
    q_ref, s_ref, c_ref = oracle.mx_quantize(x, ofmt, rule)
    torch.cuda.synchronize()
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(c), c_ref)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_mx_edge_cases_and_no_counts(fmt, ofmt):
    x = edge_case_rows(False)
    clustered = (np.float32(0.999) + np.float32(1e-5) * synth.mx_like(3, (2, 256))[1:]).astype(np.float32)
    x = np.concatenate([x, clustered], axis=0)
    q, s, c = mx.quantize_mx(dev(x), fmt, mx.RULE_FLOOR, counts=False)
    assert c is None
    q_ref, s_ref, _ = oracle.mx_quantize(x, ofmt, oracle.RULE_FLOOR)
    torch.cuda.synchronize()
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(q), q_ref)


def test_outputs_fully_written_and_deterministic():
    """Poisoned outputs are fully overwritten, and repeated runs give identical bytes."""
    x = dev(synth.activations_like(8, (512, 2048), bf16=True))
    q0, s0 = mx.quantize_token(x, mx.E4M3, mx.ROW)
    for _ in range(3):
        q = torch.full_like(q0, 0xCD)
        s = torch.full_like(s0, 0xCD)
        st = mx.fp8_quantize_token(x.data_ptr(), mx.BF16, 512, 2048, 2048, mx.ROW, mx.E4M3, q.data_ptr(),
                                   q.stride(0), s.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        assert torch.equal(q, q0) and torch.equal(s, s0)


def test_tall_inputs_beyond_65535_tile_rows():
    """More than 65535 tiles along the rows (a 2-D grid's y limit): the tile
    kernels run on 1-D grids.  Block and transposed-column codes of an
    8,388,736 x 16 bf16 tensor against the oracle."""
    rows, cols = 65536 * 128 + 128, 16
    x = synth.weights_like(123, (rows, cols), bf16=True)
    xd = dev(x)
    q, s = mx.quantize_block(xd, mx.E4M3)
    qt, st = mx.quantize_token(xd, mx.E4M3, mx.COL_T)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_block(x, oracle.E4M3, threads=16)
    assert np.array_equal(host(s), s_ref) and np.array_equal(host(q), q_ref)
    del q, q_ref
    qt_ref, st_ref = oracle.quantize_cols_t(x, oracle.E4M3, threads=16)
    assert np.array_equal(host(st), st_ref) and np.array_equal(host(qt), qt_ref)
