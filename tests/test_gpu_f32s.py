"""GPU parity of the fp32-scale variant ("FP8 w. FP32 scale"): the quantizers
must match the oracle byte for byte (codes) and bit for bit (fp32 scales); the
GEMM must stay within 2^-12 * sum|a*b| (+ 2^-22 * sum|a*b| for the rounding of
the fp32 scale product, + one bf16 rounding; on uniformly random codes a
capped count of elements may exceed it within the matrix cores' alignment
bound).  Calls go through the C ABI."""
import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import oracle
import synth
from gpu_helpers import ORACLE_THREADS, _exponent_field, adversarial_cap, assert_gemm_close, dev, dev_ld16, host
from test_gpu_quant import edge_case_rows

pytestmark = pytest.mark.gpu

FMTS = [(mx.E4M3, oracle.E4M3), (mx.E5M2, oracle.E5M2)]


def check_rows(x, fmt, ofmt):
    q, s = mx.quantize_token_f32s(dev(x), fmt, mx.ROW)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows_f32s(x, ofmt)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(q), q_ref)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shape", [(1, 16), (37, 3 * 128 + 48), (256, 512), (130, 1024 + 16)])
def test_rows_parity(fmt, ofmt, bf16, shape):
    check_rows(synth.outliers_like(shape[0] * 13 + shape[1], shape, bf16=bf16), fmt, ofmt)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("bf16", [False, True])
def test_rows_edge_cases(fmt, ofmt, bf16):
    check_rows(edge_case_rows(bf16), fmt, ofmt)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_rows_subnormal_groups(fmt, ofmt):
    """fp32 subnormal groups: subnormal scales (quotients above fmax that
    saturate) and quotients that underflow (scale 1)."""
    rng = np.random.default_rng(36)
    x = np.zeros((4, 256), np.float32)
    x[0, :128] = (rng.standard_normal(128) * 1e-39).astype(np.float32)
    x[1, :128] = (rng.integers(-5, 6, 128) * 1e-45).astype(np.float32)
    x[2, :128] = -0.0
    x[3, :128] = (rng.standard_normal(128) * 1e-41).astype(np.float32)
    x[:, 128:] = (rng.standard_normal((4, 128)) * 1e-44).astype(np.float32)
    check_rows(x, fmt, ofmt)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shape", [(16, 16), (3 * 128 + 16, 2 * 128 + 48), (512, 256)])
def test_cols_t_parity(fmt, ofmt, bf16, shape):
    x = synth.heavy_tail_like(shape[0] + 5 * shape[1], shape, bf16=bf16)
    qt, st = mx.quantize_token_f32s(dev(x), fmt, mx.COL_T)
    torch.cuda.synchronize()
    qt_ref, st_ref = oracle.quantize_cols_t_f32s(x, ofmt)
    assert np.array_equal(host(st).view(np.uint32), st_ref.view(np.uint32))
    assert np.array_equal(host(qt), qt_ref)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shape", [(1, 16), (128 + 40, 2 * 128 + 16), (300, 512)])
def test_block_parity(fmt, ofmt, bf16, shape):
    w = synth.weights_like(shape[0] * 7 + shape[1], shape, bf16=bf16)
    q, s = mx.quantize_block_f32s(dev(w), fmt)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_block_f32s(w, ofmt)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(q), q_ref)


# ------------------------------------------------------------------------ GEMM

def random_f32_scales(seed, shape):
    rng = np.random.default_rng(seed)
    return (rng.uniform(0.5, 2.0, shape) * np.exp2(rng.integers(-6, 7, shape))).astype(np.float32)


def alignment_bound(a, sa, a_fmt, b_nk, sb_cols, b_fmt):
    """The matrix cores' alignment bound (runs of 8 k, 13 bits below the run's
    largest exponent sum) with fp32 scales: sa [M][K/128], sb_cols [N][K/128]."""
    M, K = a.shape
    ea = _exponent_field(a, a_fmt)
    eb = _exponent_field(b_nk, b_fmt)
    bound = np.zeros((M, b_nk.shape[0]))
    for gi in range(K // 8):
        k0 = 8 * gi
        E = np.max(ea[:, None, k0:k0 + 8] + eb[None, :, k0:k0 + 8], axis=2)
        sc = np.abs(sa[:, k0 // 128].astype(np.float64))[:, None] * np.abs(sb_cols[:, k0 // 128].astype(np.float64))[None, :]
        bound += 8.0 * np.exp2((E - 13).astype(np.float64)) * sc
    return bound


def assert_close(y, y_ref, t_ref, bf16_out, what, hw=None):
    """The block GEMM's bound plus 2^-22 * sum|a*b| for the rounding of the fp32 scale
    product fl(sa * sb) that each K block's partial sum is multiplied by; with hw (the
    alignment bound, random codes only) a capped count of elements may exceed it."""
    hw_fn = None if hw is None else (lambda idx: hw[idx])
    assert_gemm_close(y, y_ref, t_ref, bf16_out, what, extra_rel=2.0 ** -22, hw_bound=hw_fn,
                      max_over_plain=adversarial_cap(np.size(y)) if hw is not None else 0)


def run(a, sa, a_fmt, b, sb, b_fmt, b_layout, b_scale, bf16_out):
    out = mx.gemm_f32s(dev_ld16(a), dev(sa), a_fmt, dev_ld16(b), dev(sb), b_fmt, b_layout, b_scale,
                       out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    torch.cuda.synchronize()
    return host(out)


def operands(seed, M, N, K, a_fmt, b_fmt, b_layout, b_scale):
    a = synth.random_codes(seed, (M, K), a_fmt)
    b_nk = synth.random_codes(seed + 1, (N, K), b_fmt)
    sa = random_f32_scales(seed + 2, (M, K // 128))
    if b_scale == mx.SCALE_ROW128:
        sb = random_f32_scales(seed + 3, (N, K // 128))
        sb_cols = sb
    else:
        sb = random_f32_scales(seed + 3, (-(-N // 128), K // 128))
        sb_cols = np.repeat(sb, 128, axis=0)[:N]
    b = b_nk if b_layout == mx.B_NK else np.ascontiguousarray(b_nk.T)
    sb_store = sb if (b_layout == mx.B_NK) else np.ascontiguousarray(sb.T)
    return a, sa, b, sb_store, b_nk, sb_cols


SHAPES = [(1, 16, 128), (77, 130, 384), (256 + 40, 384 + 24, 1024), (128, 128, 128 * 12), (513, 257, 256)]
MODES = [(mx.B_NK, mx.SCALE_BLOCK128), (mx.B_KN, mx.SCALE_BLOCK128), (mx.B_NK, mx.SCALE_ROW128)]


@pytest.mark.parametrize("a_fmt,b_fmt", [(0, 0), (1, 0)])
@pytest.mark.parametrize("b_layout,b_scale", MODES)
@pytest.mark.parametrize("bf16_out", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_gemm_random_codes(a_fmt, b_fmt, b_layout, b_scale, bf16_out, shape):
    M, N, K = shape
    seed = M * 17 + N * 3 + K + 10 * a_fmt + 100 * b_layout + 1000 * b_scale
    a, sa, b, sb, b_nk, sb_cols = operands(seed, M, N, K, a_fmt, b_fmt, b_layout, b_scale)
    y = run(a, sa, a_fmt, b, sb, b_fmt, b_layout, b_scale, bf16_out)
    y_ref, t_ref = oracle.gemm_f32s(a, sa, a_fmt, b, sb, b_fmt, b_layout, b_scale, threads=8)
    hw = alignment_bound(a, sa, a_fmt, b_nk, sb_cols, b_fmt)
    assert_close(y, y_ref, t_ref, bf16_out, "f32s random %s" % (shape,), hw)


@pytest.mark.parametrize("b_layout,b_scale", MODES)
def test_gemm_single_products(b_layout, b_scale):
    """One nonzero k per row of A (all K blocks of K = 512 over the rows): each
    output is one product times fl(sa * sb), so an index or scale mix-up shows
    as a wrong scale factor, well outside the 2^-22 relative bound."""
    M, N, K = 256, 256, 512
    rng = np.random.default_rng(8)
    ki = rng.integers(0, K, M)
    a = np.zeros((M, K), np.uint8)
    a[np.arange(M), ki] = rng.integers(0x30, 0x50, M)
    _, sa, b, sb, b_nk, sb_cols = operands(9, M, N, K, 0, 0, b_layout, b_scale)
    y = run(a, sa, 0, b, sb, 0, b_layout, b_scale, False)
    y_ref, t_ref = oracle.gemm_f32s(a, sa, 0, b, sb, 0, b_layout, b_scale)
    assert np.all(np.abs(y - y_ref) <= 2.0 ** -22 * t_ref)


def test_gemm_k_zero_and_ldc():
    c = torch.full((64, 48), 7.0, dtype=torch.float32, device="cuda")
    assert mx.fp8_gemm_f32s(64, 48, 0, 0, 0, 0, 0, 0, 0, 0, mx.B_NK, 0, mx.SCALE_BLOCK128, c.data_ptr(), 48,
                            mx.F32, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(c).item() == 0
    M, N, K = 100, 200, 256
    a, sa, b, sb, b_nk, sb_cols = operands(60, M, N, K, 0, 0, mx.B_NK, mx.SCALE_BLOCK128)
    c = torch.full((M, 256), -1.0, dtype=torch.float32, device="cuda")
    ad, bd, sad, sbd = dev(a), dev(b), dev(sa), dev(sb)
    assert mx.fp8_gemm_f32s(M, N, K, ad.data_ptr(), K, 0, sad.data_ptr(), bd.data_ptr(), K, 0, mx.B_NK,
                            sbd.data_ptr(), mx.SCALE_BLOCK128, c.data_ptr(), 256, mx.F32,
                            torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    ch = host(c)
    y_ref, t_ref = oracle.gemm_f32s(a, sa, 0, b, sb, 0)
    assert_close(ch[:, :N], y_ref, t_ref, False, "ldc", alignment_bound(a, sa, 0, b_nk, sb_cols, 0))
    assert np.all(ch[:, N:] == -1.0)


@pytest.mark.parametrize("bf16_out", [False, True])
def test_quantize_then_gemm_plain_bound(bf16_out):
    """fp32-scale quantizers on the GPU (bit-exact with the oracle), then the
    GEMM on those operands."""
    M, N, K = 300, 520, 1024
    x = synth.activations_like(91, (M, K), bf16=True)
    w = synth.weights_like(92, (N, K), bf16=True)
    xq, xs = mx.quantize_token_f32s(dev(x), mx.E4M3, mx.ROW)
    wq, ws = mx.quantize_block_f32s(dev(w), mx.E4M3)
    y = mx.gemm_f32s(xq, xs, mx.E4M3, wq, ws, mx.E4M3,
                     out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quantize_rows_f32s(x, oracle.E4M3)
    wq_ref, ws_ref = oracle.quantize_block_f32s(w, oracle.E4M3)
    assert np.array_equal(host(xq), xq_ref) and np.array_equal(host(xs), xs_ref)
    assert np.array_equal(host(wq), wq_ref) and np.array_equal(host(ws), ws_ref)
    y_ref, t_ref = oracle.gemm_f32s(xq_ref, xs_ref, 0, wq_ref, ws_ref, 0, threads=8)
    assert_close(host(y), y_ref, t_ref, bf16_out, "f32s quantize then gemm")


def test_fprop_1p5b_full_size():
    """The fprop shape (X 4096x1536, W 8960x1536 bf16) with fp32 scales: the
    quantizers and the GEMM compared in full."""
    d = synth.fprop1p5b()
    xq, xs = mx.quantize_token_f32s(dev(d["x"]), mx.E4M3, mx.ROW)
    wq, ws = mx.quantize_block_f32s(dev(d["w"]), mx.E4M3)
    y = mx.gemm_f32s(xq, xs, mx.E4M3, wq, ws, mx.E4M3, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quantize_rows_f32s(d["x"], oracle.E4M3, threads=ORACLE_THREADS)
    wq_ref, ws_ref = oracle.quantize_block_f32s(d["w"], oracle.E4M3, threads=ORACLE_THREADS)
    assert np.array_equal(host(xs), xs_ref) and np.array_equal(host(xq), xq_ref)
    assert np.array_equal(host(ws), ws_ref) and np.array_equal(host(wq), wq_ref)
    y_ref, t_ref = oracle.gemm_f32s(xq_ref, xs_ref, 0, wq_ref, ws_ref, 0, threads=ORACLE_THREADS)
    assert_close(host(y), y_ref, t_ref, True, "f32s fprop1p5b")
