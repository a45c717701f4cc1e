"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: every quantizer output is compared bit-for-bit with the
oracle over the whole tensor; GEMM outputs are compared on sampled elements
(tile corners, edges and random points) that the oracle computes one by one,
and checked for finiteness everywhere."""
import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import oracle
import synth
from gpu_helpers import ORACLE_THREADS, assert_gemm_close, dev, host

pytestmark = pytest.mark.gpu


def sample_points(M, N, seed, n_random=768):
    rng = np.random.default_rng(seed)
    edges_m = np.unique(np.clip(np.array([0, 1, 15, 16, 127, 128, 255, 256, M // 2, M - 129, M - 128,
                                          M - 2, M - 1]), 0, M - 1))
    edges_n = np.unique(np.clip(np.array([0, 3, 4, 15, 16, 127, 128, 255, 256, N // 2, N - 129, N - 128,
                                          N - 4, N - 1]), 0, N - 1))
    ii, jj = np.meshgrid(edges_m, edges_n, indexing="ij")
    ii = np.concatenate([ii.ravel(), rng.integers(0, M, n_random)])
    jj = np.concatenate([jj.ravel(), rng.integers(0, N, n_random)])
    return ii.astype(np.int64), jj.astype(np.int64)


def check_sampled_gemm(y_dev, a, sa, a_fmt, b, sb, b_fmt, b_layout, b_scale, bf16_out, seed, what):
    y = host(y_dev)
    assert np.isfinite(y).all(), what + ": non-finite output"
    M, N = y.shape
    ii, jj = sample_points(M, N, seed)
    y_ref, t_ref = oracle.gemm_elems(a, sa, a_fmt, b, sb, b_fmt, ii, jj, b_layout, b_scale,
                                     threads=ORACLE_THREADS)
    assert_gemm_close(y[ii, jj], y_ref, t_ref, bf16_out, what)


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
    check_sampled_gemm(y, xq_ref, xs_ref, 0, wq_ref, ws_ref, 0, 0, 0, True, 11, "fprop bf16")


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
    del gq_ref
    wq_ref, ws_ref = oracle.quantize_block(d["w"], oracle.E4M3, threads=ORACLE_THREADS)
    assert np.array_equal(host(ws), ws_ref) and np.array_equal(host(wq), wq_ref)
    check_sampled_gemm(y, host(gq), gs_ref, 1, wq_ref, ws_ref, 0, 1, 0, True, 22, "dgrad bf16")


@pytest.mark.parametrize("j", [0, 63])
def test_mx_stress_tensor(j, golden):
    x = synth.mxstress_tensor(j)
    q, s, c = mx.quantize_mx(dev(x), mx.E4M3, mx.RULE_FLOOR, counts=True)
    torch.cuda.synchronize()
    q_ref, s_ref, c_ref = oracle.mx_quantize(x, oracle.E4M3, oracle.RULE_FLOOR, threads=ORACLE_THREADS)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(c), c_ref)
    assert np.array_equal(host(q), q_ref)
    g = {r[0]: float(r[1]) for r in golden("mx_clamp_threshold.txt")}
    cnt = host(c).astype(np.int64)
    frac_normal = cnt[2048:].sum() / float(2048 * 4096)
    assert g["normal_clamped_fraction_lo"] <= frac_normal <= g["normal_clamped_fraction_hi"]
    assert cnt[:2048].sum() == 0  # 1 + N(0, 1e-3) rows sit just above a power of two


def test_mx_fprop_1p5b():
    """The fprop GEMM on MX operands: activations [4096][1536] and weights
    [8960][1536] quantized with 32-element E8M0 scales (OCP floor rule), bf16
    output; quantizers compared in full, the GEMM on samples at the plain bound."""
    d = synth.fprop1p5b()
    xq, xs, _ = mx.quantize_mx(dev(d["x"]), mx.E4M3, mx.RULE_FLOOR, counts=False)
    wq, ws, _ = mx.quantize_mx(dev(d["w"]), mx.E4M3, mx.RULE_FLOOR, counts=False)
    y = mx.mx_scaled_gemm(xq, xs, mx.E4M3, wq, ws, mx.E4M3, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    xq_ref, xs_ref, _ = oracle.mx_quantize(d["x"], oracle.E4M3, oracle.RULE_FLOOR, threads=ORACLE_THREADS)
    wq_ref, ws_ref, _ = oracle.mx_quantize(d["w"], oracle.E4M3, oracle.RULE_FLOOR, threads=ORACLE_THREADS)
    assert np.array_equal(host(xs), xs_ref) and np.array_equal(host(xq), xq_ref)
    assert np.array_equal(host(ws), ws_ref) and np.array_equal(host(wq), wq_ref)
    yh = host(y)
    assert np.isfinite(yh).all()
    ii, jj = sample_points(*yh.shape, 55)
    y_ref, t_ref = oracle.mx_gemm_elems(xq_ref, xs_ref, 0, wq_ref, ws_ref, 0, ii, jj, threads=ORACLE_THREADS)
    assert_gemm_close(yh[ii, jj], y_ref, t_ref, True, "mx fprop bf16")


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
    check_sampled_gemm(y, gq_ref, gs_ref, 1, xq_ref, xs_ref, 0, 0, 1, False, 44, "wgrad fp32")
