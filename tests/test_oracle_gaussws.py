"""Pins for the oracle's GaussWS sampler ("Gaussian Weight Sampling for
Scalable, Efficient and Stable Pseudo-Quantization Training", review page,
"What carries the argument": w_hat = w + R * max_bl(|w|) * 2^(1 - b_t) per
32x32 block, R the nearest integer to N(0,1)/2, cast to BF16).

Independent checks: numpy's own Philox4x64-10 bit generator for the uniform
bits; the closed-form probabilities of the rounded normal (math.erf) for R;
a recomputation of the formula with numpy float32 arithmetic and torch's bf16
cast from the R values; exact recovery of R where w + noise is representable."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

MASK64 = (1 << 64) - 1


def numpy_philox_block(ctr, key):
    """numpy's Philox4x64-10 output for counter `ctr` (numpy increments its
    256-bit counter before each block, so it is seeded with ctr - 1)."""
    v = sum(int(c) << (64 * i) for i, c in enumerate(ctr)) - 1
    v &= (1 << 256) - 1
    start = np.array([(v >> (64 * i)) & MASK64 for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=start)
    return bg.random_raw(4)


@pytest.mark.parametrize("key", [(0, 0), (0x0123456789ABCDEF, 0xFEDCBA9876543210), (MASK64, 7)])
def test_philox_matches_numpy(key):
    ctrs = [(1, 0, 0, 0), (0, 1, 0, 0), (12345, 678, 0, 0), (MASK64, 5, 0, 0), (3, MASK64, 9, 1)]
    for ctr in ctrs:
        assert np.array_equal(oracle.philox4x64(ctr, key), numpy_philox_block(ctr, key)), (ctr, key)


def test_r_thresholds_at_the_rounded_normal_quantiles():
    t0 = math.floor(math.erf(1 / math.sqrt(2)) * 2 ** 31 + 0.5)
    t1 = math.floor(math.erf(3 / math.sqrt(2)) * 2 ** 31 + 0.5)
    for sign in (0, 1 << 31):
        s = -1 if sign else 1
        assert oracle.gaussws_r(sign | 0) == 0
        assert oracle.gaussws_r(sign | (t0 - 1)) == 0 and oracle.gaussws_r(sign | t0) == s
        assert oracle.gaussws_r(sign | (t1 - 1)) == s and oracle.gaussws_r(sign | t1) == 2 * s
        assert oracle.gaussws_r(sign | 0x7FFFFFFF) == 2 * s


def test_r_distribution_and_independence():
    """2M draws: frequencies of -2..2 against the rounded normal's closed-form
    probabilities (chi-square, 4 degrees of freedom), and no correlation
    between neighbours along rows or columns."""
    r = oracle.gaussws_noise(2024, 11, 1024, 2048).astype(np.int64)
    n = r.size
    p0 = math.erf(1 / math.sqrt(2))
    p1 = (math.erf(3 / math.sqrt(2)) - p0) / 2
    p2 = (1 - math.erf(3 / math.sqrt(2))) / 2
    expect = np.array([p2, p1, p0, p1, p2]) * n
    counts = np.array([(r == v).sum() for v in (-2, -1, 0, 1, 2)])
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    assert chi2 < 25.0, (counts, expect, chi2)
    assert abs(counts[2] / n - 0.6827) < 0.002   # not the 0.717 of the page's unprinted approximation
    x = r.astype(np.float64)
    for a, b in ((x[:, :-1], x[:, 1:]), (x[:-1], x[1:]), (x[:, :-8], x[:, 8:])):
        c = np.corrcoef(a.ravel(), b.ravel())[0, 1]
        assert abs(c) < 0.004, c
    # different streams and seeds give different draws
    assert not np.array_equal(oracle.gaussws_noise(2024, 12, 64, 64), oracle.gaussws_noise(2024, 11, 64, 64))
    assert not np.array_equal(oracle.gaussws_noise(2025, 11, 64, 64), oracle.gaussws_noise(2024, 11, 64, 64))


def block_scales(wf, bt):
    rows, cols = wf.shape
    s = np.zeros_like(wf, dtype=np.float32)
    for i in range(0, rows, 32):
        for j in range(0, cols, 32):
            amax = np.float32(np.max(np.abs(wf[i:i + 32, j:j + 32])))
            s[i:i + 32, j:j + 32] = np.ldexp(amax, 1 - int(bt[i // 32, j // 32])).astype(np.float32)
    return s


@pytest.mark.parametrize("bf16_in", [False, True])
@pytest.mark.parametrize("shape", [(32, 32), (70, 200), (130, 96 + 8)])
def test_formula_against_numpy_and_torch(bf16_in, shape):
    """w_hat == bf16(fp32(w + R * ldexp(max_bl|w|, 1 - b_t))) recomputed here
    with numpy float32 and torch's bf16 cast, from the oracle's R."""
    rows, cols = shape
    w = synth.weights_like(rows * 3 + cols, shape, bf16=bf16_in)
    wf = synth.bf16_bits_to_f32(w) if bf16_in else w
    rng = np.random.default_rng(rows + cols)
    bt = rng.integers(2, 12, (-(-rows // 32), -(-cols // 32))).astype(np.int8)
    out = oracle.gaussws(w, bt, 99, 3)
    r = oracle.gaussws_noise(99, 3, rows, cols).astype(np.float32)
    v = (wf + r * block_scales(wf, bt)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)
    zero = r == 0
    w_bf = torch.from_numpy(wf.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out[zero], w_bf[zero])


def test_exact_recovery_of_r_and_block_indexing():
    """Block (i, j) gets amax 2^a and bitwidth b; w on the grid of its noise
    step 2^(a + 1 - b) with at most 8 significant bits, so w + noise is exact
    in bf16 and (w_hat - w) / step recovers R exactly."""
    rows, cols = 96, 128
    rng = np.random.default_rng(5)
    a = rng.integers(-3, 4, (3, 4))
    b = rng.integers(3, 7, (3, 4)).astype(np.int8)
    w = np.zeros((rows, cols), np.float32)
    step = np.zeros((rows, cols), np.float64)
    for i in range(3):
        for j in range(4):
            st = 2.0 ** (a[i, j] + 1 - b[i, j])
            k = rng.integers(-(2 ** (b[i, j] - 1)) + 3, 2 ** (b[i, j] - 1) - 3, (32, 32))
            blk = (k * st).astype(np.float32)
            blk[rng.integers(0, 32), rng.integers(0, 32)] = np.float32(2.0 ** a[i, j])
            w[32 * i:32 * i + 32, 32 * j:32 * j + 32] = blk
            step[32 * i:32 * i + 32, 32 * j:32 * j + 32] = st
    out = oracle.gaussws(w, b, 7, 1)
    w_hat = synth.bf16_bits_to_f32(out).astype(np.float64)
    rec = (w_hat - w) / step
    assert np.array_equal(rec, np.round(rec))
    assert np.array_equal(rec.astype(np.int8), oracle.gaussws_noise(7, 1, rows, cols))
