"""GPU parity of the MX GEMM (FP8 operands with one E8M0 scale per 32
elements along K) against the CPU oracle (fp64 over dequantized operands),
through the C ABI.  Bound per element: |y_gpu - y| <= 2^-12 * sum_k |a*b|
(+ one bf16 rounding for bf16 output); on uniformly random codes a capped
count of elements may exceed it within the matrix cores' alignment bound."""
import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import oracle
import synth
from gpu_helpers import (ORACLE_THREADS, adversarial_cap, assert_gemm_close, dev, dev_ld16, host,
                         alignment_bound_fn, run_mx_gemm)

pytestmark = pytest.mark.gpu

FMT_PAIRS = [(0, 0), (1, 0), (0, 1), (1, 1)]


def finite_codes(fmt):
    vals = oracle.decode(fmt, np.arange(256, dtype=np.uint8))
    return np.array([c for c in range(256) if np.isfinite(vals[c])], dtype=np.uint8)


@pytest.mark.parametrize("a_fmt,b_fmt", FMT_PAIRS)
def test_outer_products_with_chunk_scales_exact(a_fmt, b_fmt):
    """One nonzero k per row pair, in the fifth 32-wide chunk: C[i][j] =
    dec(a_i) 2^(sa_i) dec(b_j) 2^(sb_j) exactly.  The other chunks' scale bytes
    are extreme, so reading a neighbouring chunk's byte shows."""
    ca, cb = finite_codes(a_fmt), finite_codes(b_fmt)
    M, N, K = len(ca), len(cb), 256
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((N, K), np.uint8)
    a[:, 4 * 32 + 5] = ca
    b[:, 4 * 32 + 5] = cb
    rng = np.random.default_rng(5)
    sa = np.full((M, K // 32), 250, np.uint8)
    sb = np.full((N, K // 32), 3, np.uint8)
    sa[:, 4] = rng.integers(123, 132, M)
    sb[:, 4] = rng.integers(123, 132, N)
    y = run_mx_gemm(a, sa, a_fmt, b, sb, b_fmt, False)
    ref = np.outer(oracle.decode(a_fmt, ca) * np.exp2(sa[:, 4].astype(np.float64) - 127),
                   oracle.decode(b_fmt, cb) * np.exp2(sb[:, 4].astype(np.float64) - 127))
    assert np.array_equal(y.astype(np.float64), ref)


def test_every_chunk_scale_is_read_from_its_own_byte():
    """A row i of A holds one nonzero code at k_i (all chunks of K = 512 over
    the rows); B is dense.  Each output is one product scaled by sa[i][k_i/32]
    and sb[j][k_i/32], so any mix-up of chunk, row or half of the scale bytes
    changes it by a power of two."""
    M, N, K = 256, 192, 512
    rng = np.random.default_rng(9)
    ki = rng.permutation(np.arange(K))[:M]
    a = np.zeros((M, K), np.uint8)
    a[np.arange(M), ki] = rng.integers(0x30, 0x50, M)  # E4M3 values near 1
    b = rng.integers(0x30, 0x50, (N, K)).astype(np.uint8)
    sa = rng.integers(118, 137, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(118, 137, (N, K // 32)).astype(np.uint8)
    y = run_mx_gemm(a, sa, 0, b, sb, 0, False)
    y_ref, t_ref = oracle.mx_gemm(a, sa, 0, b, sb, 0)
    assert np.array_equal(y.astype(np.float64), y_ref)


SHAPES = [(1, 16, 128), (77, 130, 384), (256 + 40, 384 + 24, 1024), (128, 128, 128 * 12), (513, 257, 256)]


@pytest.mark.parametrize("a_fmt,b_fmt", FMT_PAIRS)
@pytest.mark.parametrize("bf16_out", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_random_codes_parity(a_fmt, b_fmt, bf16_out, shape):
    M, N, K = shape
    seed = M * 37 + N * 5 + K + 100 * a_fmt + 10 * b_fmt
    a = synth.random_codes(seed, (M, K), a_fmt)
    b = synth.random_codes(seed + 1, (N, K), b_fmt)
    sa = synth.random_scale_bytes(seed + 2, (M, K // 32))
    sb = synth.random_scale_bytes(seed + 3, (N, K // 32))
    y = run_mx_gemm(a, sa, a_fmt, b, sb, b_fmt, bf16_out)
    y_ref, t_ref = oracle.mx_gemm(a, sa, a_fmt, b, sb, b_fmt, threads=8)
    hb = alignment_bound_fn(a, sa, a_fmt, b, sb, b_fmt, mx_scales=True)
    assert_gemm_close(y, y_ref, t_ref, bf16_out, "mx random codes %s" % (shape,), hw_bound=hb,
                      max_over_plain=adversarial_cap(y.size))


def test_k_zero_writes_zeros():
    c = torch.full((64, 48), 7.0, dtype=torch.float32, device="cuda")
    st = mx.mx_gemm(64, 48, 0, 0, 0, 0, 0, 0, 0, 0, 0, c.data_ptr(), 48, mx.F32,
                    torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(c).item() == 0


def test_ldc_larger_than_n_leaves_padding():
    M, N, K = 100, 200, 256
    a = synth.random_codes(15, (M, K), 0)
    b = synth.random_codes(16, (N, K), 0)
    sa = synth.random_scale_bytes(17, (M, K // 32))
    sb = synth.random_scale_bytes(18, (N, K // 32))
    c = torch.full((M, 256), -1.0, dtype=torch.float32, device="cuda")
    ad, bd, sad, sbd = dev(a), dev(b), dev(sa), dev(sb)
    st = mx.mx_gemm(M, N, K, ad.data_ptr(), K, 0, sad.data_ptr(), bd.data_ptr(), K, 0, sbd.data_ptr(),
                    c.data_ptr(), 256, mx.F32, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    ch = host(c)
    y_ref, t_ref = oracle.mx_gemm(a, sa, 0, b, sb, 0)
    assert_gemm_close(ch[:, :N], y_ref, t_ref, False, "ldc", hw_bound=alignment_bound_fn(a, sa, 0, b, sb, 0, mx_scales=True),
                      max_over_plain=adversarial_cap(M * N))
    assert np.all(ch[:, N:] == -1.0)


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("a_fmt,b_fmt", [(0, 0), (1, 0)])
def test_quantize_then_gemm_strict_bound(x_dtype, a_fmt, b_fmt):
    """mx_quantize on the GPU (bit-exact with the oracle), then mx_gemm on those
    bytes, held to the plain 2^-12 * sum|a*b| bound."""
    M, N, K = 300, 520, 1024
    bf = x_dtype == "bf16"
    x = synth.activations_like(71, (M, K), bf16=bf)
    w = synth.weights_like(72, (N, K), bf16=bf)
    xq, xs, _ = mx.quantize_mx(dev(x), a_fmt, mx.RULE_FLOOR, counts=False)
    wq, ws, _ = mx.quantize_mx(dev(w), b_fmt, mx.RULE_FLOOR, counts=False)
    y = mx.mx_scaled_gemm(xq, xs, a_fmt, wq, ws, b_fmt)
    torch.cuda.synchronize()
    xq_ref, xs_ref, _ = oracle.mx_quantize(x, a_fmt, oracle.RULE_FLOOR)
    wq_ref, ws_ref, _ = oracle.mx_quantize(w, b_fmt, oracle.RULE_FLOOR)
    assert np.array_equal(host(xq), xq_ref) and np.array_equal(host(xs), xs_ref)
    assert np.array_equal(host(wq), wq_ref) and np.array_equal(host(ws), ws_ref)
    y_ref, t_ref = oracle.mx_gemm(xq_ref, xs_ref, a_fmt, wq_ref, ws_ref, b_fmt, threads=8)
    assert_gemm_close(host(y), y_ref, t_ref, False, "mx quantize then gemm")


@pytest.mark.parametrize("bf16_out", [False, True])
def test_short_last_round_as_quadrants(bf16_out):
    """17 x 16 cells of 256x256 on 256 CUs: the last 16 cells run as 128x128
    quadrants after the 256x256 tiles, in the same launch.  Quadrant rows
    compared in full, the rest on samples."""
    M, N, K = 256 * 16 + 100, 256 * 16 - 30, 256
    seed = 177 + bf16_out
    a = synth.random_codes(seed, (M, K), 0)
    b = synth.random_codes(seed + 1, (N, K), 1)
    sa = synth.random_scale_bytes(seed + 2, (M, K // 32))
    sb = synth.random_scale_bytes(seed + 3, (N, K // 32))
    y = run_mx_gemm(a, sa, 0, b, sb, 1, bf16_out)
    assert np.isfinite(y).all()
    r0 = 256 * 16
    y_ref, t_ref = oracle.mx_gemm(a[r0:], sa[r0:], 0, b, sb, 1, threads=8)
    hb = alignment_bound_fn(a[r0:], sa[r0:], 0, b, sb, 1, mx_scales=True)
    assert_gemm_close(y[r0:], y_ref, t_ref, bf16_out, "quadrant rows", hw_bound=hb,
                      max_over_plain=adversarial_cap(y_ref.size))
    rng = np.random.default_rng(seed)
    ii = np.concatenate([rng.integers(r0 - 256, r0, 2048), rng.integers(0, r0, 512)])
    jj = rng.integers(0, N, ii.size)
    y_s, t_s = oracle.mx_gemm_elems(a, sa, 0, b, sb, 1, ii, jj, threads=8)
    hb_s = alignment_bound_fn(a, sa, 0, b, sb, 1, mx_scales=True, ii=ii, jj=jj)
    assert_gemm_close(y[ii, jj], y_s, t_s, bf16_out, "sampled", hw_bound=hb_s, max_over_plain=adversarial_cap(ii.size))


def test_strided_operands():
    """Row pitches above K for A and B (views into wider buffers)."""
    M, N, K = 200, 300, 640
    a = synth.random_codes(31, (M, K), 1)
    b = synth.random_codes(32, (N, K), 0)
    sa = synth.random_scale_bytes(33, (M, K // 32))
    sb = synth.random_scale_bytes(34, (N, K // 32))
    y = mx.mx_scaled_gemm(dev(a, pitch=K + 48), dev(sa), 1, dev(b, pitch=K + 16), dev(sb), 0)
    torch.cuda.synchronize()
    y_ref, t_ref = oracle.mx_gemm(a, sa, 1, b, sb, 0, threads=8)
    assert_gemm_close(host(y), y_ref, t_ref, False, "strided", hw_bound=alignment_bound_fn(a, sa, 1, b, sb, 0, mx_scales=True),
                      max_over_plain=adversarial_cap(M * N))
