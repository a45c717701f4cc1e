"""Pins for the oracle's FP8 codec (decode, saturating RNE encode).

Each check compares the oracle with something it does not share code with:
torch's float8 decode tables (a library routine), the format facts printed on
the pages (tests/golden/), and an independent nearest-code search encoder
written here.
"""
import numpy as np
import pytest
import torch

import oracle
from refcodec import nearest_code_encoder, structured_f32, torch_decode_table

FMTS = [(oracle.E4M3, torch.float8_e4m3fn, 448.0), (oracle.E5M2, torch.float8_e5m2, 57344.0)]


def golden_facts(golden):
    return {r[0]: r[1:] for r in golden("fp8_format_facts.txt")}


# ---------------------------------------------------------------------- decode pins

@pytest.mark.parametrize("fmt,tdt,fmax", FMTS)
def test_decode_matches_torch_tables(fmt, tdt, fmax):
    ours = oracle.decode(fmt, np.arange(256, dtype=np.uint8))
    ref = torch_decode_table(tdt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # sign of zero: 0x80 decodes to -0.0
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_decode_format_facts(golden):
    f = golden_facts(golden)
    e4 = oracle.decode(oracle.E4M3, np.arange(256, dtype=np.uint8))
    e5 = oracle.decode(oracle.E5M2, np.arange(256, dtype=np.uint8))
    assert sorted(np.nonzero(np.isnan(e4))[0].tolist()) == [int(c, 16) for c in f["e4m3_nan_codes"]]
    assert not np.isinf(e4).any()
    assert e4[int(f["e4m3_max_code"][0], 16)] == float(f["e4m3_max"][0]) == np.nanmax(e4)
    assert e4[int(f["e4m3_min_normal_code"][0], 16)] == float(f["e4m3_min_normal"][0])
    assert e4[int(f["e4m3_min_subnormal_code"][0], 16)] == float(f["e4m3_min_subnormal"][0])
    assert sorted(np.nonzero(np.isinf(e5))[0].tolist()) == [int(c, 16) for c in f["e5m2_inf_codes"]]
    assert sorted(np.nonzero(np.isnan(e5))[0].tolist()) == [int(c, 16) for c in f["e5m2_nan_codes"]]
    assert e5[int(f["e5m2_max_code"][0], 16)] == float(f["e5m2_max"][0]) == np.nanmax(e5[np.isfinite(e5)])
    assert e5[int(f["e5m2_min_subnormal_code"][0], 16)] == float(f["e5m2_min_subnormal"][0])


def test_e4m3_code_gaps_match_fig5(golden):
    g = {r[0]: (float(r[1]), float(r[2])) for r in golden("e4m3_code_gaps.txt")}
    vals = oracle.decode(oracle.E4M3, np.arange(0x08, 0x7F, dtype=np.uint8))  # positive normals
    firsts, lasts = [], []
    for band in range(1, 15):  # full bands E = 1 .. 14 (E = 15 lacks its NaN slot)
        v = vals[(band - 1) * 8:(band - 1) * 8 + 9]  # 1.000 .. 2.000 of the band
        gaps = (v[1:] - v[:-1]) / v[:-1]
        assert np.all(np.diff(gaps) < 0)
        firsts.append(gaps[0])
        lasts.append(gaps[-1])
    assert np.allclose(firsts, g["first_gap"][0], atol=g["first_gap"][1])
    assert np.allclose(lasts, g["last_gap"][0], atol=g["last_gap"][1])


# ---------------------------------------------------------------------- encode pins

@pytest.mark.parametrize("fmt,tdt,fmax", FMTS)
def test_encode_roundtrip_all_codes(fmt, tdt, fmax):
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode(fmt, codes)
    ok = ~np.isnan(vals) & ~np.isinf(vals)
    assert np.array_equal(oracle.encode(fmt, vals[ok]), codes[ok])


@pytest.mark.parametrize("fmt,tdt,fmax", FMTS)
def test_encode_all_bf16_patterns_vs_nearest_search(fmt, tdt, fmax):
    bits = np.arange(65536, dtype=np.uint32) << 16
    with np.errstate(invalid="ignore"):
        x = bits.view(np.float32).astype(np.float64)
    ours = oracle.encode(fmt, x)
    ref = nearest_code_encoder(x, tdt, fmax)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7F) == 0x7F)


@pytest.mark.parametrize("fmt,tdt,fmax", FMTS)
def test_encode_structured_f32_vs_nearest_search(fmt, tdt, fmax):
    x = structured_f32().astype(np.float64)
    ours = oracle.encode(fmt, x)
    ref = nearest_code_encoder(x, tdt, fmax)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(x[i], hex(ours[i]), hex(ref[i])) for i in bad[:5]]


@pytest.mark.parametrize("fmt,tdt,fmax", FMTS)
def test_encode_random_f32_patterns_vs_nearest_search(fmt, tdt, fmax):
    bits = np.random.default_rng(7).integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    with np.errstate(invalid="ignore"):
        x = bits.view(np.float32).astype(np.float64)
    fin = np.isfinite(x)
    ours = oracle.encode(fmt, x[fin])
    ref = nearest_code_encoder(x[fin], tdt, fmax)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("fmt,tdt,fmax", FMTS)
def test_encode_range_entry_matches_array_entry(fmt, tdt, fmax):
    start = 0x3B000000  # a span crossing the subnormal / normal boundaries of both formats
    n = 1 << 20
    x = (np.arange(n, dtype=np.uint64) + start).astype(np.uint32).view(np.float32).astype(np.float64)
    assert np.array_equal(oracle.encode_f32_range(fmt, start, n), nearest_code_encoder(x, tdt, fmax))


@pytest.mark.parametrize("fmt,tdt,fmax", FMTS)
def test_encode_agrees_with_torch_cast_in_range(fmt, tdt, fmax):
    # torch's CPU cast rounds to nearest-even but does not saturate, so compare inside +-fmax.
    x32 = structured_f32()
    x32 = x32[np.abs(x32) <= fmax]
    ref = torch.from_numpy(x32).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode(fmt, x32.astype(np.float64)), ref)


@pytest.mark.parametrize("fmt,tdt,fmax", FMTS)
def test_encode_saturates(fmt, tdt, fmax):
    top = 0x7E if fmt == oracle.E4M3 else 0x7B
    xs = [fmax * (1 + 2.0 ** -k) for k in range(1, 50)] + [fmax * 2, 1e30, 3.0e38]
    assert np.all(oracle.encode(fmt, np.array(xs)) == top)
    assert np.all(oracle.encode(fmt, -np.array(xs)) == (top | 0x80))


def test_encode_e4m3_top_binade_ties():
    # quantum 32 in [256, 512): 464 is a tie between 448 (m=6, even) and 480 (NaN slot)
    assert oracle.encode(oracle.E4M3, np.array([464.0]))[0] == 0x7E
    assert oracle.encode(oracle.E4M3, np.array([432.0]))[0] == 0x7E  # tie 416/448 -> even m=6
    assert oracle.encode(oracle.E4M3, np.array([400.0]))[0] == 0x7C  # tie 384/416 -> even m=4


def test_encode_sign_of_zero_and_specials():
    e4 = oracle.encode(oracle.E4M3, np.array([0.0, -0.0, -1e-30, np.nan, np.inf, -np.inf]))
    assert list(e4) == [0x00, 0x80, 0x80, 0x7F, 0x7E, 0xFE]
    e5 = oracle.encode(oracle.E5M2, np.array([0.0, -0.0, -1e-30, np.inf, -np.inf]))
    assert list(e5) == [0x00, 0x80, 0x80, 0x7C, 0xFC]
