"""Pins for the oracle's fp32-scale variant ("FP8 with an FP32 scale", named on
the review page of "A Comprehensive FP8 Training Recipe for Reasoning-Enhanced
Language Models" as a Table 4 variant; read here as: scale = amax / fmax in
IEEE fp32, 1 where that quotient is zero, code = saturating cast of the fp32
quotient x / scale).

Independent checks: numpy's own float32 division for the scale and the
quotient, the nearest-code search over torch's decode table for the cast, the
special case of power-of-two scales (which must reproduce the pinned E8M0
quantizers and GEMM), exact rational sums for the GEMM and numpy matmul."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from refcodec import nearest_code_encoder

FMAX = {oracle.E4M3: 448.0, oracle.E5M2: 57344.0}
TDT = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}


def f32_values(x):
    return synth.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x.astype(np.float32)


def bf_quantize(vals_f32, fmt):
    """One group: numpy float32 scale and quotient, then the nearest-code search."""
    amax = np.max(np.abs(vals_f32)) if vals_f32.size else np.float32(0)
    s = np.float32(amax) / np.float32(FMAX[fmt])
    s = np.float32(1.0) if s == 0 else s
    with np.errstate(over="ignore", divide="ignore"):
        v = vals_f32 / s
    return nearest_code_encoder(v.astype(np.float64), TDT[fmt], FMAX[fmt]), s


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_scale_is_ieee_single_division(fmt):
    rng = np.random.default_rng(3)
    bits = rng.integers(1, 0x7F7FFFFF, 20000, dtype=np.uint32)
    amaxes = np.concatenate([bits.view(np.float32), np.float32([1e-40, 2e-43, 448.0, 57344.0, 3.4e38])])
    for a in amaxes:
        q = np.float32(a) / np.float32(FMAX[fmt])
        assert oracle.scale_f32(fmt, a) == (q if q != 0 else np.float32(1.0)), a
    # a quotient that rounds to zero is replaced by 1, like an all-zero group
    assert oracle.scale_f32(fmt, 0.0) == 1.0
    assert oracle.scale_f32(fmt, 1e-45) == 1.0 and np.float32(1e-45) / np.float32(FMAX[fmt]) == 0


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("bf16", [False, True])
def test_rows_vs_bruteforce(fmt, bf16):
    x = synth.outliers_like(31, (6, 3 * 128 + 48), bf16=bf16)
    xf = f32_values(x)
    q, s = oracle.quantize_rows_f32s(x, fmt)
    for r in range(x.shape[0]):
        for g, c0 in enumerate(range(0, x.shape[1], 128)):
            qr, sr = bf_quantize(xf[r, c0:c0 + 128], fmt)
            assert s[r, g] == sr
            assert np.array_equal(q[r, c0:c0 + 128], qr)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_tiny_and_subnormal_groups(fmt):
    """Groups of fp32 subnormals: scales that are themselves subnormal (few
    significant bits, quotients above fmax that saturate) and scales whose
    quotient underflows (replaced by 1)."""
    rng = np.random.default_rng(36)
    x = np.zeros((4, 256), np.float32)
    x[0, :128] = (rng.standard_normal(128) * 1e-39).astype(np.float32)
    x[1, :128] = (rng.integers(-5, 6, 128) * 1e-45).astype(np.float32)
    x[2, :128] = -0.0
    x[3, :128] = (rng.standard_normal(128) * 1e-41).astype(np.float32)
    x[:, 128:] = (rng.standard_normal((4, 128)) * 1e-44).astype(np.float32)
    q, s = oracle.quantize_rows_f32s(x, fmt)
    for r in range(4):
        for g in range(2):
            qr, sr = bf_quantize(x[r, 128 * g:128 * (g + 1)], fmt)
            assert s[r, g] == sr
            assert np.array_equal(q[r, 128 * g:128 * (g + 1)], qr)
    assert np.all(q[2, :128] == 0x80)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_cols_t_vs_bruteforce(fmt):
    x = synth.heavy_tail_like(32, (2 * 128 + 80, 6), bf16=True)
    xf = f32_values(x)
    qt, st = oracle.quantize_cols_t_f32s(x, fmt)
    for c in range(x.shape[1]):
        for t, r0 in enumerate(range(0, x.shape[0], 128)):
            qr, sr = bf_quantize(xf[r0:r0 + 128, c], fmt)
            assert st[c, t] == sr
            assert np.array_equal(qt[c, r0:r0 + 128], qr)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_block_vs_bruteforce(fmt):
    w = synth.weights_like(33, (128 + 40, 2 * 128 + 16), bf16=False)
    w[5, 200] = 0.7
    q, s = oracle.quantize_block_f32s(w, fmt)
    for i, r0 in enumerate(range(0, w.shape[0], 128)):
        for j, c0 in enumerate(range(0, w.shape[1], 128)):
            tile = w[r0:r0 + 128, c0:c0 + 128]
            qr, sr = bf_quantize(tile.reshape(-1), fmt)
            assert s[i, j] == sr
            assert np.array_equal(q[r0:r0 + 128, c0:c0 + 128].reshape(-1), qr)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_power_of_two_scales_reduce_to_e8m0(fmt):
    """Groups whose amax is fmax * 2^k get the scale 2^k exactly, and then the
    codes of the round-up E8M0 quantizer (a special case of both rules)."""
    rng = np.random.default_rng(34)
    rows, cols = 24, 256
    x = (rng.standard_normal((rows, cols)) * 0.3).astype(np.float32)
    k = rng.integers(-20, 20, (rows, 2))
    for r in range(rows):
        for g in range(2):
            grp = x[r, 128 * g:128 * (g + 1)]
            grp *= np.float32(FMAX[fmt] * 2.0 ** k[r, g]) / np.max(np.abs(grp)) * np.float32(0.999)
            grp[rng.integers(0, 128)] = np.float32(FMAX[fmt] * 2.0 ** k[r, g]) * (1 if rng.random() < 0.5 else -1)
    q, s = oracle.quantize_rows_f32s(x, fmt)
    q8, s8 = oracle.quantize_rows(x, fmt)
    assert np.array_equal(s, np.exp2(k).astype(np.float32))
    assert np.array_equal(s8.astype(np.int64) - 127, k)
    assert np.array_equal(q, q8)


def test_quotient_rounding_matters():
    """Elements whose fp32 quotient x / s lands exactly on an E4M3 rounding tie
    while x * (1 / s) lands one fp32 ulp off it: the oracle must take the
    division (a mistake that multiplies by the reciprocal changes these codes)."""
    rng = np.random.default_rng(35)
    ties = np.float32(1.0) + (2 * np.arange(8, dtype=np.float32) + 1) / np.float32(16)
    rows = []
    while len(rows) < 16:
        amax = np.float32(rng.uniform(0.5, 1000.0))
        s = amax / np.float32(448.0)
        xs = (ties * s).astype(np.float32)
        div = xs / s
        mul = xs * (np.float32(1.0) / s)
        pick = (div == ties) & (mul != ties)
        if pick.any():
            row = np.zeros(128, np.float32)
            row[0] = amax
            row[1:1 + pick.sum()] = xs[pick]
            rows.append(row)
    x = np.stack(rows)
    q, sc = oracle.quantize_rows_f32s(x, oracle.E4M3)
    q_div = nearest_code_encoder((x / sc[:, :1]).astype(np.float64), TDT[0], 448.0)
    q_mul = nearest_code_encoder((x * (np.float32(1) / sc[:, :1])).astype(np.float64), TDT[0], 448.0)
    assert np.array_equal(q, q_div)
    assert not np.array_equal(q, q_mul)


# ------------------------------------------------------------------------ GEMM

def exact_value(code, fmt):
    mb, eb = (3, 4) if fmt == oracle.E4M3 else (2, 5)
    bias = (1 << (eb - 1)) - 1
    s = -1 if code & 0x80 else 1
    E = (code >> mb) & ((1 << eb) - 1)
    m = code & ((1 << mb) - 1)
    if E == 0:
        return s * Fraction(m, 1 << mb) * Fraction(2) ** (1 - bias)
    return s * (1 + Fraction(m, 1 << mb)) * Fraction(2) ** (E - bias)


def random_f32_scales(seed, shape):
    rng = np.random.default_rng(seed)
    return (rng.uniform(0.5, 2.0, shape) * np.exp2(rng.integers(-8, 8, shape))).astype(np.float32)


@pytest.mark.parametrize("a_fmt,b_fmt", [(0, 0), (1, 0)])
@pytest.mark.parametrize("b_layout,b_scale", [(0, 0), (1, 0), (0, 1)])
def test_gemm_tiny_exact_rational(a_fmt, b_fmt, b_layout, b_scale):
    M, N, K = 3, 4, 256
    a = synth.random_codes(41, (M, K), a_fmt)
    b_nk = synth.random_codes(42, (N, K), b_fmt)
    sa = random_f32_scales(43, (M, K // 128))
    sb = random_f32_scales(44, (N, K // 128) if b_scale == 1 else (1, K // 128))
    b = b_nk if b_layout == 0 else np.ascontiguousarray(b_nk.T)
    sb_store = sb if (b_layout == 0 or b_scale == 1) else np.ascontiguousarray(sb.T)
    y, t = oracle.gemm_f32s(a, sa, a_fmt, b, sb_store, b_fmt, b_layout, b_scale)
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                sbk = sb[j, k // 128] if b_scale == 1 else sb[0, k // 128]
                p = (exact_value(int(a[i, k]), a_fmt) * Fraction(float(sa[i, k // 128]))
                     * exact_value(int(b_nk[j, k]), b_fmt) * Fraction(float(sbk)))
                acc += p
                mag += abs(p)
            bound = mag * K * Fraction(2) ** -52  # one product rounding + K-term fp64 sum
            assert abs(Fraction(y[i, j]) - acc) <= bound
            assert abs(Fraction(t[i, j]) - mag) <= bound


def test_gemm_power_of_two_scales_equal_byte_gemm():
    M, N, K = 20, 3 * 128 + 8, 3 * 128
    a = synth.random_codes(45, (M, K), 1)
    b = synth.random_codes(46, (N, K), 0)
    sa8 = synth.random_scale_bytes(47, (M, K // 128))
    sb8 = synth.random_scale_bytes(48, (-(-N // 128), K // 128))
    y8, t8 = oracle.gemm(a, sa8, 1, b, sb8, 0)
    sa = np.exp2(sa8.astype(np.float64) - 127).astype(np.float32)
    sb = np.exp2(sb8.astype(np.float64) - 127).astype(np.float32)
    y, t = oracle.gemm_f32s(a, sa, 1, b, sb, 0)
    assert np.array_equal(y, y8) and np.array_equal(t, t8)


@pytest.mark.parametrize("b_layout,b_scale", [(0, 0), (1, 0), (0, 1)])
def test_gemm_matches_numpy_matmul(b_layout, b_scale):
    M, N, K = 30, 2 * 128 + 24, 3 * 128
    a = synth.random_codes(49, (M, K), 0)
    b_nk = synth.random_codes(50, (N, K), 0)
    sa = random_f32_scales(51, (M, K // 128))
    if b_scale == 0:
        sb = random_f32_scales(52, (-(-N // 128), K // 128))
        sb_full = np.repeat(np.repeat(sb, 128, axis=0)[:N], 128, axis=1)
    else:
        sb = random_f32_scales(52, (N, K // 128))
        sb_full = np.repeat(sb, 128, axis=1)
    tdec = lambda c, f: torch.from_numpy(c).view(TDT[f]).to(torch.float64).numpy()
    A = tdec(a, 0) * np.repeat(sa, 128, axis=1).astype(np.float64)
    B = tdec(b_nk, 0) * sb_full.astype(np.float64)
    ref = A @ B.T
    mag = np.abs(A) @ np.abs(B).T
    b_store = b_nk if b_layout == 0 else np.ascontiguousarray(b_nk.T)
    sb_store = sb if (b_layout == 0 or b_scale == 1) else np.ascontiguousarray(sb.T)
    y, t = oracle.gemm_f32s(a, sa, 0, b_store, sb_store, 0, b_layout, b_scale, threads=4)
    assert np.all(np.abs(y - ref) <= 2 * K * 2.0 ** -52 * mag)
    assert np.allclose(t, mag, rtol=2 * K * 2.0 ** -52, atol=0)
    ii = np.array([0, 5, 29, 11], np.int64)
    jj = np.array([0, 270, 128, 3], np.int64)
    ye, te = oracle.gemm_f32s_elems(a, sa, 0, b_store, sb_store, 0, ii, jj, b_layout, b_scale)
    assert np.array_equal(ye, y[ii, jj]) and np.array_equal(te, t[ii, jj])
