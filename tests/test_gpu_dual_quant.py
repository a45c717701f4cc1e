"""GPU parity of the two-orientation quantizers against the CPU oracle,
through the C ABI: fp8_quantize_token_dual must give byte-for-byte the oracle's
row groups and transposed column groups of the same input, and
fp8_quantize_block_dual the oracle's 128x128 block codes, their transpose and
the transposed scale grid."""
import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import oracle
import synth
from gpu_helpers import ORACLE_THREADS, assert_gemm_close, dev, host
from test_gpu_quant import edge_case_rows

pytestmark = pytest.mark.gpu

FMTS = [(mx.E4M3, oracle.E4M3), (mx.E5M2, oracle.E5M2)]
SHAPES = [(16, 16), (48, 128 + 16), (3 * 128 + 16, 2 * 128 + 48), (512, 256), (256 + 32, 1024 + 16)]


def check_token_dual(x, fmt, ofmt):
    q, s, qt, st = mx.quantize_token_dual(dev(x), fmt)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows(x, ofmt)
    qt_ref, st_ref = oracle.quantize_cols_t(x, ofmt)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(st), st_ref)
    assert np.array_equal(host(qt), qt_ref)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_token_dual_parity(fmt, ofmt, bf16, shape):
    check_token_dual(synth.outliers_like(shape[0] * 5 + shape[1], shape, bf16=bf16), fmt, ofmt)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("bf16", [False, True])
def test_token_dual_edge_cases(fmt, ofmt, bf16):
    """The degenerate groups along rows (16 x 256) and down columns (256 x 16)."""
    x = edge_case_rows(False)
    rows = np.concatenate([x, x[::-1] * np.float32(0.5)]).astype(np.float32)
    cols = np.ascontiguousarray(rows.T)
    for a in (rows, cols):
        check_token_dual(synth.to_bf16_bits(a) if bf16 else a, fmt, ofmt)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_token_dual_leading_dimensions(fmt, ofmt):
    R, C = 96, 384
    x = synth.activations_like(6, (R, C), bf16=True)
    xd = dev(x, pitch=400)
    q = torch.full((R, 512), 0xCD, dtype=torch.uint8, device="cuda")
    qt = torch.full((C, 128), 0xCD, dtype=torch.uint8, device="cuda")
    s = torch.empty((R, 3), dtype=torch.uint8, device="cuda")
    st = torch.empty((C, 1), dtype=torch.uint8, device="cuda")
    r = mx.fp8_quantize_token_dual(xd.data_ptr(), mx.BF16, R, C, 400, fmt, q.data_ptr(), 512, s.data_ptr(),
                                   qt.data_ptr(), 128, st.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert r == 0
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows(x, ofmt)
    qt_ref, st_ref = oracle.quantize_cols_t(x, ofmt)
    qh, qth = host(q), host(qt)
    assert np.array_equal(qh[:, :C], q_ref) and np.all(qh[:, C:] == 0xCD)
    assert np.array_equal(qth[:, :R], qt_ref) and np.all(qth[:, R:] == 0xCD)
    assert np.array_equal(host(s), s_ref) and np.array_equal(host(st), st_ref)


def check_block_dual(w, fmt, ofmt):
    q, s, qt, st = mx.quantize_block_dual(dev(w), fmt)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_block(w, ofmt)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(st), s_ref.T)
    assert np.array_equal(host(qt), q_ref.T)
    return q_ref, s_ref


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shape", [(16, 16), (128, 128), (128 + 48, 2 * 128 + 16), (304, 512), (512, 48)])
def test_block_dual_parity(fmt, ofmt, bf16, shape):
    check_block_dual(synth.weights_like(shape[0] * 11 + shape[1], shape, bf16=bf16), fmt, ofmt)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_block_dual_edge_cases(fmt, ofmt):
    x = edge_case_rows(False)
    w = np.zeros((256, 272), np.float32)
    w[:8, :256] = x
    w[130:138, 16:] = x[::-1]
    w[200, 3] = 1e-41
    w[255, 271] = -3e38
    check_block_dual(w, fmt, ofmt)


def test_dgrad_through_transposed_weight():
    """dX = dY * W with W [out][in]: the transposed codes make W^T an [N][K]
    operand; both B layouts give results within the bound of the oracle."""
    T, O, I = 256, 384, 512
    w = synth.weights_like(81, (O, I), bf16=True)
    dy = synth.gradients_like(82, (T, O), bf16=True)
    q, s, qt, st = mx.quantize_block_dual(dev(w), mx.E4M3)
    gq, gs = mx.quantize_token(dev(dy), mx.E5M2, mx.ROW)
    y_kn = mx.block_scaled_gemm(gq, gs, mx.E5M2, q, s, mx.E4M3, mx.B_KN, mx.SCALE_BLOCK128)
    y_nk = mx.block_scaled_gemm(gq, gs, mx.E5M2, qt, st, mx.E4M3, mx.B_NK, mx.SCALE_BLOCK128)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_block(w, oracle.E4M3)
    gq_ref, gs_ref = oracle.quantize_rows(dy, oracle.E5M2)
    assert np.array_equal(host(qt), q_ref.T) and np.array_equal(host(gq), gq_ref)
    y_ref, t_ref = oracle.gemm(gq_ref, gs_ref, 1, q_ref, s_ref, 0, oracle.B_KN, oracle.B_SCALE_BLOCK)
    assert_gemm_close(host(y_kn), y_ref, t_ref, False, "dgrad KN")
    assert_gemm_close(host(y_nk), y_ref, t_ref, False, "dgrad NK via W^T")


def test_wgrad_activation_both_orientations_full_size():
    """X 16384 x 4096 bf16 (t(3) x 0.5): the row codes (forward) and the
    transposed column codes (weight gradient) of one read, whole tensors."""
    x = synth.wgrad()["x"]
    q, s, qt, st = mx.quantize_token_dual(dev(x), mx.E4M3)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows(x, oracle.E4M3, threads=ORACLE_THREADS)
    assert np.array_equal(host(s), s_ref) and np.array_equal(host(q), q_ref)
    del q_ref, q
    qt_ref, st_ref = oracle.quantize_cols_t(x, oracle.E4M3, threads=ORACLE_THREADS)
    assert np.array_equal(host(st), st_ref) and np.array_equal(host(qt), qt_ref)


def test_dgrad_weight_with_transpose_full_size():
    """W 18944 x 3584 bf16 N(0, 0.015): block codes and their transpose, whole tensors."""
    w = synth.dgrad7b(rows=16)["w"]
    q, s, qt, st = mx.quantize_block_dual(dev(w), mx.E4M3)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_block(w, oracle.E4M3, threads=ORACLE_THREADS)
    assert np.array_equal(host(s), s_ref) and np.array_equal(host(st), s_ref.T)
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(qt), q_ref.T)
