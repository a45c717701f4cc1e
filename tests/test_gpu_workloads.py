"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: every quantizer output is compared bit-for-bit with the
oracle over the whole tensor, and every GEMM output element is compared with
the oracle's fp64 sum over the same codes (the whole product, computed on the
host's threads), at the plain 2^-12 * sum|a*b| bound plus one bf16 rounding
where the output is bf16."""
import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import oracle
import synth
from gpu_helpers import ORACLE_THREADS, assert_gemm_close, dev, host

pytestmark = pytest.mark.gpu


def check_full_gemm(y_dev, a, sa, a_fmt, b, sb, b_fmt, b_layout, b_scale, bf16_out, what, y32_dev=None):
    """Every output element against the oracle's fp64 product over the same codes; with
    y32_dev (the same GEMM with fp32 output) also every element at the pure
    2^-12 * sum|a*b| bound, without the bf16 rounding term."""
    y = host(y_dev)
    y_ref, t_ref = oracle.gemm(a, sa, a_fmt, b, sb, b_fmt, b_layout, b_scale, threads=ORACLE_THREADS)
    assert_gemm_close(y, y_ref, t_ref, bf16_out, what)
    if y32_dev is not None:
        assert_gemm_close(host(y32_dev), y_ref, t_ref, False, what.replace("bf16", "fp32"))


def test_tiny_reference_full():
    d = synth.tiny()
    xq, xs = mx.quantize_token(dev(d["x"]), mx.E4M3, mx.ROW)
    wq, ws = mx.quantize_block(dev(d["w"]), mx.E4M3)
    y = mx.block_scaled_gemm(xq, xs, mx.E4M3, wq, ws, mx.E4M3, mx.B_NK, mx.SCALE_BLOCK128)
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quantize_rows(d["x"], oracle.E4M3)
    wq_ref, ws_ref = oracle.quantize_block(d["w"], oracle.E4M3)
    assert np.array_equal(host(xq), xq_ref) and np.array_equal(host(xs), xs_ref)
    assert np.array_equal(host(wq), wq_ref) and np.array_equal(host(ws), ws_ref)
    y_ref, t_ref = oracle.gemm(xq_ref, xs_ref, 0, wq_ref, ws_ref, 0, threads=ORACLE_THREADS)
    assert_gemm_close(host(y), y_ref, t_ref, False, "tiny")


def test_fprop_1p5b():
    d = synth.fprop1p5b()
    xq, xs = mx.quantize_token(dev(d["x"]), mx.E4M3, mx.ROW)
    wq, ws = mx.quantize_block(dev(d["w"]), mx.E4M3)
    y = mx.block_scaled_gemm(xq, xs, mx.E4M3, wq, ws, mx.E4M3, mx.B_NK, mx.SCALE_BLOCK128,
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quantize_rows(d["x"], oracle.E4M3, threads=ORACLE_THREADS)
    wq_ref, ws_ref = oracle.quantize_block(d["w"], oracle.E4M3, threads=ORACLE_THREADS)
    assert np.array_equal(host(xs), xs_ref) and np.array_equal(host(xq), xq_ref)
    assert np.array_equal(host(ws), ws_ref) and np.array_equal(host(wq), wq_ref)
    y32 = mx.block_scaled_gemm(xq, xs, mx.E4M3, wq, ws, mx.E4M3, mx.B_NK, mx.SCALE_BLOCK128)
    torch.cuda.synchronize()
    check_full_gemm(y, xq_ref, xs_ref, 0, wq_ref, ws_ref, 0, 0, 0, True, "fprop1p5b bf16", y32)


def test_dgrad_7b():
    d = synth.dgrad7b()
    gq, gs = mx.quantize_token(dev(d["dy"]), mx.E5M2, mx.ROW)
    wq, ws = mx.quantize_block(dev(d["w"]), mx.E4M3)
    # dX = dY * W with W stored [K = 18944][N = 3584]
    y = mx.block_scaled_gemm(gq, gs, mx.E5M2, wq, ws, mx.E4M3, mx.B_KN, mx.SCALE_BLOCK128,
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    gq_ref, gs_ref = oracle.quantize_rows(d["dy"], oracle.E5M2, threads=ORACLE_THREADS)
    assert np.array_equal(host(gs), gs_ref) and np.array_equal(host(gq), gq_ref)
    wq_ref, ws_ref = oracle.quantize_block(d["w"], oracle.E4M3, threads=ORACLE_THREADS)
    assert np.array_equal(host(ws), ws_ref) and np.array_equal(host(wq), wq_ref)
    y32 = mx.block_scaled_gemm(gq, gs, mx.E5M2, wq, ws, mx.E4M3, mx.B_KN, mx.SCALE_BLOCK128)
    torch.cuda.synchronize()
    check_full_gemm(y, gq_ref, gs_ref, 1, wq_ref, ws_ref, 0, 1, 0, True, "dgrad7b bf16", y32)


@pytest.mark.parametrize("group", range(4))
def test_mx_stress_tensors(group, golden):
    """All 64 tensors of the MX clamping stress (16 per case): codes, scale bytes and
    clamp counts bit-exact; per tensor, the strict clamp fraction of the N(0,1) rows
    inside the golden band and none in the clustered 1 + N(0,1e-3) rows."""
    g = {r[0]: float(r[1]) for r in golden("mx_clamp_threshold.txt")}
    for j in range(16 * group, 16 * group + 16):
        x = synth.mxstress_tensor(j)
        q, s, c = mx.quantize_mx(dev(x), mx.E4M3, mx.RULE_FLOOR, counts=True)
        torch.cuda.synchronize()
        q_ref, s_ref, c_ref = oracle.mx_quantize(x, oracle.E4M3, oracle.RULE_FLOOR, threads=ORACLE_THREADS)
        assert np.array_equal(host(s), s_ref), "scales of tensor %d" % j
        assert np.array_equal(host(c), c_ref), "clamp counts of tensor %d" % j
        assert np.array_equal(host(q), q_ref), "codes of tensor %d" % j
        cnt = c_ref.astype(np.int64)
        frac_normal = cnt[2048:].sum() / float(2048 * 4096)
        assert g["normal_clamped_fraction_lo"] <= frac_normal <= g["normal_clamped_fraction_hi"], j
        assert cnt[:2048].sum() == 0, j  # 1 + N(0, 1e-3) rows sit just above a power of two


def test_mx_fprop_1p5b():
    """The fprop GEMM on MX operands: activations [4096][1536] and weights
    [8960][1536] quantized with 32-element E8M0 scales (OCP floor rule), bf16
    output; quantizers and the GEMM compared in full at the plain bound."""
    d = synth.fprop1p5b()
    xq, xs, _ = mx.quantize_mx(dev(d["x"]), mx.E4M3, mx.RULE_FLOOR, counts=False)
    wq, ws, _ = mx.quantize_mx(dev(d["w"]), mx.E4M3, mx.RULE_FLOOR, counts=False)
    y = mx.mx_scaled_gemm(xq, xs, mx.E4M3, wq, ws, mx.E4M3, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    xq_ref, xs_ref, _ = oracle.mx_quantize(d["x"], oracle.E4M3, oracle.RULE_FLOOR, threads=ORACLE_THREADS)
    wq_ref, ws_ref, _ = oracle.mx_quantize(d["w"], oracle.E4M3, oracle.RULE_FLOOR, threads=ORACLE_THREADS)
    assert np.array_equal(host(xs), xs_ref) and np.array_equal(host(xq), xq_ref)
    assert np.array_equal(host(ws), ws_ref) and np.array_equal(host(wq), wq_ref)
    y32 = mx.mx_scaled_gemm(xq, xs, mx.E4M3, wq, ws, mx.E4M3)
    torch.cuda.synchronize()
    y_ref, t_ref = oracle.mx_gemm(xq_ref, xs_ref, 0, wq_ref, ws_ref, 0, threads=ORACLE_THREADS)
    assert_gemm_close(host(y), y_ref, t_ref, True, "mx fprop1p5b bf16")
    assert_gemm_close(host(y32), y_ref, t_ref, False, "mx fprop1p5b fp32")


def test_wgrad():
    d = synth.wgrad()
    xq, xs = mx.quantize_token(dev(d["x"]), mx.E4M3, mx.COL_T)     # [4096][16384], [4096][128]
    gq, gs = mx.quantize_token(dev(d["dy"]), mx.E5M2, mx.COL_T)
    # dW[o][i] = sum_t dY[t][o] X[t][i]: A = dY^T (E5M2), B = X^T stored [N][K] with per-row scales
    y = mx.block_scaled_gemm(gq, gs, mx.E5M2, xq, xs, mx.E4M3, mx.B_NK, mx.SCALE_ROW128)
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quantize_cols_t(d["x"], oracle.E4M3, threads=ORACLE_THREADS)
    assert np.array_equal(host(xs), xs_ref) and np.array_equal(host(xq), xq_ref)
    gq_ref, gs_ref = oracle.quantize_cols_t(d["dy"], oracle.E5M2, threads=ORACLE_THREADS)
    assert np.array_equal(host(gs), gs_ref) and np.array_equal(host(gq), gq_ref)
    check_full_gemm(y, gq_ref, gs_ref, 1, xq_ref, xs_ref, 0, 0, 1, False, "wgrad fp32")
