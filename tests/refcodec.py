"""Reference pieces for tests, written independently of the oracle's C code.

``nearest_code_encoder`` encodes by searching torch's float8 decode table for
the nearest finite code (ties to the even code, saturation to +-max, sign
kept); ``structured_f32`` enumerates fp32 values that exercise every rounding
case of both FP8 formats.
"""
import numpy as np
import torch


def torch_decode_table(tdt):
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(tdt).to(torch.float64).numpy()


def nearest_code_encoder(x, tdt, fmax):
    """Independent encoder: nearest finite code by search over torch's decode table,
    ties to the code with an even mantissa (even code integer), saturation to +-fmax,
    sign kept (also for results that round to zero)."""
    table = torch_decode_table(tdt)
    pos_codes = np.array([c for c in range(0x80) if np.isfinite(table[c])], dtype=np.int64)
    pos_vals = table[pos_codes]
    order = np.argsort(pos_vals, kind="stable")
    pos_codes, pos_vals = pos_codes[order], pos_vals[order]
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    a_c = np.minimum(a, fmax)
    hi = np.clip(np.searchsorted(pos_vals, a_c, side="left"), 0, len(pos_vals) - 1)
    lo = np.clip(hi - 1, 0, len(pos_vals) - 1)
    d_lo = np.abs(a_c - pos_vals[lo])
    d_hi = np.abs(pos_vals[hi] - a_c)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (pos_codes[hi] % 2 == 0))
    code = np.where(pick_hi, pos_codes[hi], pos_codes[lo]).astype(np.uint8)
    code = code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    code = np.where(np.isnan(x), (0x7F | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8), code)
    if tdt == torch.float8_e5m2:
        code = np.where(np.isinf(x), np.where(x > 0, 0x7C, 0xFC).astype(np.uint8), code)
    return code.astype(np.uint8)


def structured_f32(exp_lo=127 - 30, exp_hi=127 + 20):
    """All exponents in range x both signs x every top-12 mantissa pattern x six low-bit
    patterns (exact, round bit, sticky variants)."""
    lows = np.array([0, 1, 0x3FF, 0x400, 0x401, 0x7FF], dtype=np.uint32)
    e = np.arange(exp_lo, exp_hi + 1, dtype=np.uint32)
    m = np.arange(4096, dtype=np.uint32) << 11
    bits = (e[:, None, None] << 23) | m[None, :, None] | lows[None, None, :]
    bits = bits.reshape(-1)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    return bits.view(np.float32)


