"""Pins for the oracle's block-scaled GEMM.

Independent checks: exact rational arithmetic (Python fractions) on tiny
matrices, exact outer products of single codes, the effect of one scale byte,
the equivalence of B's storage layouts and scale modes, and a numpy fp64
matmul over torch-decoded operands (library routines).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

TDT = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}


def torch_dec(codes, fmt):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(TDT[fmt]).to(torch.float64).numpy()


def exact_value(code, fmt):
    """Exact rational value of a finite FP8 code, from its bit fields."""
    mb, eb = (3, 4) if fmt == oracle.E4M3 else (2, 5)
    bias = (1 << (eb - 1)) - 1
    s = -1 if code & 0x80 else 1
    E = (code >> mb) & ((1 << eb) - 1)
    m = code & ((1 << mb) - 1)
    if E == 0:
        return s * Fraction(m, 1 << mb) * Fraction(2) ** (1 - bias)
    return s * (1 + Fraction(m, 1 << mb)) * Fraction(2) ** (E - bias)


@pytest.mark.parametrize("a_fmt,b_fmt", [(0, 0), (1, 0), (1, 1)])
@pytest.mark.parametrize("K", [128, 256, 384])
def test_tiny_exact_rational(a_fmt, b_fmt, K):
    M, N = 3, 4
    a = synth.random_codes(21 + K, (M, K), a_fmt)
    b = synth.random_codes(22 + K, (N, K), b_fmt)
    sa = synth.random_scale_bytes(23 + K, (M, K // 128), 100, 150)
    sb = synth.random_scale_bytes(24 + K, (1, K // 128), 100, 150)
    y, t = oracle.gemm(a, sa, a_fmt, b, sb, b_fmt)
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                p = (exact_value(int(a[i, k]), a_fmt) * Fraction(2) ** (int(sa[i, k // 128]) - 127)
                     * exact_value(int(b[j, k]), b_fmt) * Fraction(2) ** (int(sb[0, k // 128]) - 127))
                acc += p
                mag += abs(p)
            # fp64 recursive summation of K terms: |error| <= (K - 1) * 2^-53 * sum|terms|
            bound = mag * (K - 1) * Fraction(2) ** -53
            assert abs(Fraction(y[i, j]) - acc) <= bound
            assert abs(Fraction(t[i, j]) - mag) <= bound


@pytest.mark.parametrize("a_fmt,b_fmt", [(0, 0), (1, 0), (1, 1)])
def test_outer_products_of_single_codes_exact(a_fmt, b_fmt):
    def finite_codes(fmt):
        return [c for c in range(256) if np.isfinite(torch_dec(np.array([c], np.uint8), fmt)[0])]
    ca, cb = finite_codes(a_fmt), finite_codes(b_fmt)
    a = np.zeros((len(ca), 128), np.uint8)
    b = np.zeros((len(cb), 128), np.uint8)
    a[:, 0] = ca
    b[:, 0] = cb
    sa = np.full((len(ca), 1), 127, np.uint8)
    sb = np.full((-(-len(cb) // 128), 1), 127, np.uint8)
    y, _ = oracle.gemm(a, sa, a_fmt, b, sb, b_fmt)
    ref = np.outer(torch_dec(np.array(ca, np.uint8), a_fmt), torch_dec(np.array(cb, np.uint8), b_fmt))
    assert np.array_equal(y, ref)


def test_scale_byte_bump_doubles_one_block():
    M, N, K = 2, 3, 384
    a = synth.random_codes(31, (M, K), 0)
    b = synth.random_codes(32, (N, K), 0)
    sa = synth.random_scale_bytes(33, (M, K // 128))
    sb = synth.random_scale_bytes(34, (1, K // 128))
    y0, _ = oracle.gemm(a, sa, 0, b, sb, 0)
    sa2 = sa.copy()
    sa2[1, 2] += 1
    y1, _ = oracle.gemm(a, sa2, 0, b, sb, 0)
    # contribution of row 1, K block 2, computed with the block isolated
    a_blk = a.copy()
    a_blk[:, :256] = 0
    yb, _ = oracle.gemm(a_blk, sa, 0, b, sb, 0)
    assert np.array_equal(y1[0], y0[0])
    assert np.allclose(y1[1] - y0[1], yb[1], rtol=2.0 ** -45, atol=0)


def test_layouts_and_scale_modes_agree():
    M, N, K = 5, 2 * 128 + 16, 3 * 128
    a = synth.random_codes(41, (M, K), 1)
    b_nk = synth.random_codes(42, (N, K), 0)
    sa = synth.random_scale_bytes(43, (M, K // 128))
    sb_blk = synth.random_scale_bytes(44, (-(-N // 128), K // 128))
    y_nk, t_nk = oracle.gemm(a, sa, 1, b_nk, sb_blk, 0, oracle.B_NK, oracle.B_SCALE_BLOCK)
    # KN storage of the same B, with tile scales laid out [K/128][N/128]
    y_kn, t_kn = oracle.gemm(a, sa, 1, np.ascontiguousarray(b_nk.T), np.ascontiguousarray(sb_blk.T), 0,
                             oracle.B_KN, oracle.B_SCALE_BLOCK)
    assert np.array_equal(y_nk, y_kn) and np.array_equal(t_nk, t_kn)
    # per-row scales equal to the tile scale of each row's tile
    sb_row = np.repeat(sb_blk, 128, axis=0)[:N]
    y_row, _ = oracle.gemm(a, sa, 1, b_nk, sb_row, 0, oracle.B_NK, oracle.B_SCALE_ROW)
    assert np.array_equal(y_nk, y_row)


@pytest.mark.parametrize("b_layout,b_scale", [(0, 0), (1, 0), (0, 1)])
def test_matches_numpy_matmul_of_torch_decoded(b_layout, b_scale):
    M, N, K = 40, 3 * 128 + 8, 4 * 128
    a = synth.random_codes(51, (M, K), 0)
    b_nk = synth.random_codes(52, (N, K), 1)
    sa = synth.random_scale_bytes(53, (M, K // 128))
    if b_scale == 0:
        sb = synth.random_scale_bytes(54, (-(-N // 128), K // 128))
        sb_full = np.repeat(np.repeat(sb, 128, axis=0)[:N], 128, axis=1)
    else:
        sb = synth.random_scale_bytes(54, (N, K // 128))
        sb_full = np.repeat(sb, 128, axis=1)
    sa_full = np.repeat(sa, 128, axis=1)
    A = torch_dec(a, 0) * 2.0 ** (sa_full.astype(np.float64) - 127)
    B = torch_dec(b_nk, 1) * 2.0 ** (sb_full.astype(np.float64) - 127)
    ref = A @ B.T
    b_store = b_nk if b_layout == 0 else np.ascontiguousarray(b_nk.T)
    sb_store = sb if (b_layout == 0 or b_scale == 1) else np.ascontiguousarray(sb.T)
    y, t = oracle.gemm(a, sa, 0, b_store, sb_store, 1, b_layout, b_scale, threads=4)
    mag = np.abs(A) @ np.abs(B).T
    # two fp64 summations of K terms each: 2 * K * 2^-53 relative to sum|a*b|
    assert np.all(np.abs(y - ref) <= 2 * K * 2.0 ** -53 * mag)
    assert np.allclose(t, mag, rtol=2 * K * 2.0 ** -53, atol=0)
    assert np.all(t >= np.abs(y))
    # element entry point agrees with the full product
    ii = np.array([0, 7, 39, 20], np.int64)
    jj = np.array([0, 385, 128, 200], np.int64)
    ye, te = oracle.gemm_elems(a, sa, 0, b_store, sb_store, 1, ii, jj, b_layout, b_scale)
    assert np.array_equal(ye, y[ii, jj]) and np.array_equal(te, t[ii, jj])


# ---------------------------------------------------------------- MX GEMM
# Pins for oracle.mx_gemm: operands scaled per 32-element block along K
# ("Characterization and Mitigation of Training Instabilities in Microscaling
# Formats", "What carries the argument").

@pytest.mark.parametrize("a_fmt,b_fmt", [(0, 0), (1, 0), (0, 1)])
@pytest.mark.parametrize("K", [32, 96, 256])
def test_mx_tiny_exact_rational(a_fmt, b_fmt, K):
    M, N = 3, 4
    a = synth.random_codes(61 + K, (M, K), a_fmt)
    b = synth.random_codes(62 + K, (N, K), b_fmt)
    sa = synth.random_scale_bytes(63 + K, (M, K // 32), 100, 150)
    sb = synth.random_scale_bytes(64 + K, (N, K // 32), 100, 150)
    y, t = oracle.mx_gemm(a, sa, a_fmt, b, sb, b_fmt)
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                p = (exact_value(int(a[i, k]), a_fmt) * Fraction(2) ** (int(sa[i, k // 32]) - 127)
                     * exact_value(int(b[j, k]), b_fmt) * Fraction(2) ** (int(sb[j, k // 32]) - 127))
                acc += p
                mag += abs(p)
            bound = mag * (K - 1) * Fraction(2) ** -53
            assert abs(Fraction(y[i, j]) - acc) <= bound
            assert abs(Fraction(t[i, j]) - mag) <= bound


def test_mx_scale_byte_bump_doubles_one_32_block():
    M, N, K = 2, 3, 256
    a = synth.random_codes(71, (M, K), 0)
    b = synth.random_codes(72, (N, K), 0)
    sa = synth.random_scale_bytes(73, (M, K // 32))
    sb = synth.random_scale_bytes(74, (N, K // 32))
    y0, _ = oracle.mx_gemm(a, sa, 0, b, sb, 0)
    sb2 = sb.copy()
    sb2[2, 5] += 1  # column 2, k in [160, 192)
    y1, _ = oracle.mx_gemm(a, sa, 0, b, sb2, 0)
    a_blk = np.zeros_like(a)
    a_blk[:, 160:192] = a[:, 160:192]
    yb, _ = oracle.mx_gemm(a_blk, sa, 0, b, sb, 0)
    assert np.array_equal(y1[:, :2], y0[:, :2])
    assert np.allclose(y1[:, 2] - y0[:, 2], yb[:, 2], rtol=2.0 ** -45, atol=0)


def test_mx_matches_numpy_matmul_of_torch_decoded():
    M, N, K = 24, 40, 320
    a = synth.random_codes(81, (M, K), 1)
    b = synth.random_codes(82, (N, K), 0)
    sa = synth.random_scale_bytes(83, (M, K // 32))
    sb = synth.random_scale_bytes(84, (N, K // 32))
    A = torch_dec(a, 1) * 2.0 ** (np.repeat(sa, 32, axis=1).astype(np.float64) - 127)
    B = torch_dec(b, 0) * 2.0 ** (np.repeat(sb, 32, axis=1).astype(np.float64) - 127)
    y, t = oracle.mx_gemm(a, sa, 1, b, sb, 0, threads=4)
    mag = np.abs(A) @ np.abs(B).T
    assert np.allclose(y, A @ B.T, rtol=0, atol=K * 2.0 ** -52 * mag.max())
    assert np.allclose(t, mag, rtol=K * 2.0 ** -52, atol=0)
    yi, ti = oracle.mx_gemm_elems(a, sa, 1, b, sb, 0, np.array([0, 5, 23]), np.array([39, 0, 17]))
    assert np.array_equal(yi, y[[0, 5, 23], [39, 0, 17]]) and np.array_equal(ti, t[[0, 5, 23], [39, 0, 17]])


def test_mx_with_uniform_128_scales_equals_block_gemm():
    """Four equal 32-block scales per 128 block give the per-(row, 128) GEMM."""
    M, N, K = 6, 10, 384
    a = synth.random_codes(91, (M, K), 0)
    b = synth.random_codes(92, (N, K), 1)
    sa128 = synth.random_scale_bytes(93, (M, K // 128))
    sb128 = synth.random_scale_bytes(94, (N, K // 128))
    y_mx, t_mx = oracle.mx_gemm(a, np.repeat(sa128, 4, axis=1), 0, b, np.repeat(sb128, 4, axis=1), 1)
    y_bs, t_bs = oracle.gemm(a, sa128, 0, b, sb128, 1, oracle.B_NK, oracle.B_SCALE_ROW)
    assert np.array_equal(y_mx, y_bs) and np.array_equal(t_mx, t_bs)
