"""Pins for the oracle's scale rules and quantizers.

Independent checks: closed-form scale exponents, the invariants the pages state
(round-up scales never leave the FP8 range; the MX floor rule clamps above
0.875 of the binade top), a hand-derived worked example (tests/golden/), and a
brute-force quantizer written here from scratch (exponent search with Python
fractions, nearest-code search over torch's decode table).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from refcodec import nearest_code_encoder

FMAX = {oracle.E4M3: 448.0, oracle.E5M2: 57344.0}
TDT = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}


# -------------------------------------------------------------------- scale rules

@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_ceil_rule_closed_forms(fmt):
    fmax = FMAX[fmt]
    for k in range(-100, 100):
        assert oracle.scale_exp_ceil(fmt, fmax * 2.0 ** k) == k
        assert oracle.scale_exp_ceil(fmt, fmax * 2.0 ** k * (1 + 2.0 ** -23)) == k + 1
        assert oracle.scale_exp_ceil(fmt, fmax * 2.0 ** k * 0.5 * (1 + 2.0 ** -23)) == k
    assert oracle.scale_exp_ceil(fmt, 0.0) == -127
    assert oracle.scale_exp_ceil(fmt, 1e-45) == -127  # fp32 subnormal, below fmax * 2^-127


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_ceil_rule_invariants_random(fmt):
    fmax = FMAX[fmt]
    rng = np.random.default_rng(3)
    amax = np.abs(rng.standard_normal(20000) * np.exp(rng.uniform(-60, 60, 20000))).astype(np.float32)
    for a in amax.astype(np.float64):
        e = oracle.scale_exp_ceil(fmt, a)
        assert a <= fmax * 2.0 ** e  # never leaves the range
        assert e == -127 or a > fmax * 2.0 ** (e - 1)  # and is the smallest such power


@pytest.mark.parametrize("fmt,emax_elem", [(oracle.E4M3, 8), (oracle.E5M2, 15)])
def test_floor_rule_binade(fmt, emax_elem, golden):
    g = {r[0]: float(r[1]) for r in golden("mx_clamp_threshold.txt")}
    rng = np.random.default_rng(4)
    amax = np.abs(rng.standard_normal(20000) * np.exp(rng.uniform(-40, 40, 20000))).astype(np.float32)
    for a in amax.astype(np.float64):
        X = oracle.scale_exp_floor(fmt, a)
        s = a * 2.0 ** -X
        assert 2.0 ** emax_elem <= s < 2.0 ** (emax_elem + 1)
        if fmt == oracle.E4M3:
            assert g["scaled_binade_lo"] <= s < g["scaled_binade_hi"]
        # the two rules differ by one exactly when the scaled amax clears fmax
        e = oracle.scale_exp_ceil(fmt, a)
        assert e - X in (0, 1)
        assert (e - X == 1) == (s > FMAX[fmt])
    assert oracle.scale_exp_floor(fmt, 0.0) == -127


def test_floor_rule_clamp_threshold_is_0875(golden):
    g = {r[0]: float(r[1]) for r in golden("mx_clamp_threshold.txt")}
    thr = g["threshold_fraction"]
    for p in range(-20, 20):
        at = thr * 2.0 ** (p + 1)  # significand exactly 1.75
        above = at * (1 + 2.0 ** -20)
        x_at = np.array([[at] + [0.0] * 31], dtype=np.float32)
        x_above = np.array([[above] + [0.0] * 31], dtype=np.float32)
        _, _, c_at = oracle.mx_quantize(x_at, oracle.E4M3, oracle.RULE_FLOOR)
        _, _, c_above = oracle.mx_quantize(x_above, oracle.E4M3, oracle.RULE_FLOOR)
        assert c_at[0, 0] == 0 and c_above[0, 0] == 1


# ---------------------------------------------------------------- worked example

def test_token_group_worked_example(golden):
    rows = golden("token_group_example.txt")
    scale = int(rows[0][1])
    x = np.zeros((1, 128), np.float32)
    expect = {}
    for r in rows[1:]:
        x[0, int(r[0])] = np.float32(float(r[1]))
        expect[int(r[0])] = int(r[2], 16)
    q, s = oracle.quantize_rows(x, oracle.E4M3)
    assert s[0, 0] == scale
    for i, c in expect.items():
        assert q[0, i] == c, (i, hex(q[0, i]), hex(c))
    assert np.all(q[0, len(expect):] == 0)


# ------------------------------------------------------- brute-force quantizers

def bf_exponent_ceil(amax, fmax):
    """Smallest integer e with amax <= fmax * 2^e, searched with exact rationals."""
    a, f = Fraction(float(amax)), Fraction(float(fmax))
    for e in range(-127, 128):
        if a <= f * (Fraction(2) ** e):
            return e
    return 127


def bf_exponent_floor(amax, fmax):
    if amax == 0:
        return -127
    a = Fraction(float(amax))
    p = 0
    while Fraction(2) ** p > a:
        p -= 1
    while Fraction(2) ** (p + 1) <= a:
        p += 1
    emax = 0
    while Fraction(2) ** (emax + 1) <= Fraction(float(fmax)):
        emax += 1
    return max(-127, min(127, p - emax))


def widen(x):
    return synth.bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def bf_groups(xv, fmt, group_axis_len, groups, rule="ceil"):
    """Quantize a list of groups (index arrays into xv) with the brute-force pieces."""
    fmax = FMAX[fmt]
    q = np.zeros(xv.shape, np.uint8)
    s = []
    cnt = []
    for idx in groups:
        vals = xv[idx]
        amax = np.max(np.abs(vals)) if vals.size else 0.0
        e = bf_exponent_ceil(amax, fmax) if rule == "ceil" else bf_exponent_floor(amax, fmax)
        scaled = vals * 2.0 ** -e
        q[idx] = nearest_code_encoder(scaled, TDT[fmt], fmax)
        s.append(e + 127)
        cnt.append(int(np.sum(np.abs(scaled) > fmax)))
    return q, np.array(s, np.uint8), np.array(cnt, np.uint8)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("bf16", [False, True])
def test_rows_vs_bruteforce(fmt, bf16):
    x = synth.outliers_like(11, (5, 3 * 128 + 48), bf16=bf16)  # ragged last group
    xv = widen(x)
    rows, cols = x.shape
    groups = [(np.full(min(128, cols - c0), r), np.arange(c0, min(c0 + 128, cols)))
              for r in range(rows) for c0 in range(0, cols, 128)]
    q_ref, s_ref, _ = bf_groups(xv, fmt, 128, groups)
    q, s = oracle.quantize_rows(x, fmt)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(s.reshape(-1), s_ref)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_cols_t_vs_bruteforce(fmt):
    x = synth.heavy_tail_like(12, (2 * 128 + 80, 6), bf16=True)  # ragged token tail
    xv = widen(x)
    rows, cols = x.shape
    groups = [(np.arange(r0, min(r0 + 128, rows)), np.full(min(128, rows - r0), c))
              for c in range(cols) for r0 in range(0, rows, 128)]
    q_ref, s_ref, _ = bf_groups(xv, fmt, 128, groups)
    qt, st = oracle.quantize_cols_t(x, fmt)
    assert np.array_equal(qt, q_ref.T)
    assert np.array_equal(st.reshape(-1), s_ref)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_block_vs_bruteforce(fmt):
    x = synth.weights_like(13, (128 + 40, 2 * 128 + 16), bf16=False)
    x[0, 0] = 3.0  # one large element: its tile gets a different scale
    xv = widen(x)
    rows, cols = x.shape
    groups = []
    for r0 in range(0, rows, 128):
        for c0 in range(0, cols, 128):
            rr, cc = np.meshgrid(np.arange(r0, min(r0 + 128, rows)), np.arange(c0, min(c0 + 128, cols)),
                                 indexing="ij")
            groups.append((rr.reshape(-1), cc.reshape(-1)))
    q_ref, s_ref, _ = bf_groups(xv, fmt, 128, groups)
    q, s = oracle.quantize_block(x, fmt)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(s.reshape(-1), s_ref)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("rule", ["floor", "ceil"])
def test_mx_vs_bruteforce(fmt, rule):
    x = synth.mx_like(14, (8, 5 * 32))
    x[1, 3] = 0.9995  # a block whose amax significand exceeds 1.75 -> clamps under floor
    x[1, :32] = np.float32(0.9995) + x[1, :32] * np.float32(1e-6)
    xv = widen(x)
    rows, cols = x.shape
    groups = [(np.full(32, r), np.arange(c0, c0 + 32)) for r in range(rows) for c0 in range(0, cols, 32)]
    q_ref, s_ref, c_ref = bf_groups(xv, fmt, 32, groups, rule=rule)
    q, s, c = oracle.mx_quantize(x, fmt, oracle.RULE_FLOOR if rule == "floor" else oracle.RULE_CEIL)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(s.reshape(-1), s_ref)
    assert np.array_equal(c.reshape(-1), c_ref)
    if rule == "ceil":
        assert np.all(c == 0)  # round-up scales never clamp


# ------------------------------------------------------------ page-level behaviour

@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_roundup_scales_use_top_binade_and_never_saturate(fmt):
    x = synth.activations_like(15, (64, 1024), bf16=True)
    q, s = oracle.quantize_rows(x, fmt)
    xv = widen(x).reshape(64, 8, 128)
    e = s.astype(np.int64) - 127
    scaled = np.abs(xv) * 2.0 ** -e[:, :, None]
    fmax = FMAX[fmt]
    assert np.all(scaled <= fmax)
    amax_scaled = scaled.max(axis=2)
    assert np.all((amax_scaled > fmax / 2) & (amax_scaled <= fmax))
    # dequantized values within half a quantum of the inputs (relative 2^-4 / 2^-3 for normals)
    deq = oracle.decode(fmt, q).reshape(64, 8, 128) * 2.0 ** e[:, :, None]
    mb = 3 if fmt == oracle.E4M3 else 2
    normal = scaled >= (2.0 ** -6 if fmt == oracle.E4M3 else 2.0 ** -14)
    rel = np.abs(deq - xv)[normal] / np.abs(xv)[normal]
    assert rel.max() <= 2.0 ** -(mb + 1)


def test_mx_clustered_blocks_collapse_and_normal_blocks_clamp_about_one_percent(golden):
    g = {r[0]: float(r[1]) for r in golden("mx_clamp_threshold.txt")}
    x = synth.mx_like(16, (512, 1024))
    q, s, c = oracle.mx_quantize(x, oracle.E4M3, oracle.RULE_FLOOR)
    top = q[:256]
    # 1 + N(0, 1e-3) sits just above a power of two: every element lands on one code
    # (256 after scaling: 0x78) and nothing clamps
    assert np.all(top == 0x78) and np.all(c[:256] == 0)
    frac = c[256:].sum() / float(256 * 1024)
    assert g["normal_clamped_fraction_lo"] <= frac <= g["normal_clamped_fraction_hi"], frac
    # a tight cluster just below a power of two: the whole block clamps to the last bin
    y = (np.float32(0.999) + np.float32(1e-5) * synth.mx_like(17, (4, 64))[2:]).astype(np.float32)
    qy, sy, cy = oracle.mx_quantize(y, oracle.E4M3, oracle.RULE_FLOOR)
    assert np.all(qy == 0x7E) and np.all(cy == 32)
