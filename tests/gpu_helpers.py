"""Helpers for the GPU parity tests: host <-> device marshalling and the
tolerances of the block-scaled GEMM."""
import json
import os

import numpy as np
import torch

import mx_block_scaled_x128_amd as mx

ORACLE_THREADS = min(16, os.cpu_count() or 1)


def dev(a, pitch=None):
    """numpy float32 / bf16-bits (uint16) / uint8 array -> CUDA tensor.  Dense by default;
    with `pitch`, a 2-D view of a wider buffer (row pitch `pitch` elements)."""
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    if pitch is not None and pitch != a.shape[1]:
        buf = torch.zeros((a.shape[0], pitch), dtype=t.dtype)
        buf[:, :a.shape[1]] = t
        return buf.cuda()[:, :a.shape[1]]
    return t.cuda()


def dev_ld16(a):
    """2-D array -> CUDA view whose row pitch is the next multiple of 16 elements."""
    return dev(a, pitch=(a.shape[1] + 15) // 16 * 16)


def host(t):
    """CUDA tensor (possibly a strided view) -> numpy (bf16 as float32)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def gemm_tolerance(y_ref, t_ref, bf16_out, extra_rel=0.0):
    """Per-element bound: 2^-12 * sum|a*b| (plus extra_rel * sum|a*b| where a variant
    adds a documented term) for fp32 output; one extra bf16 rounding (unit roundoff
    2^-8 of a value within that bound of y) for bf16 output."""
    tol = (2.0 ** -12 + extra_rel) * t_ref
    if bf16_out:
        tol = tol + 2.0 ** -8 * (np.abs(y_ref) + tol)
    return tol


def record_ratio(what, ratio, n, over=0):
    """Appends the largest err / bound of a comparison, its element count and the count
    above the bound as a JSON line to the file named by MXFP8_RATIO_LOG, if set, tagged
    with the running test."""
    path = os.environ.get("MXFP8_RATIO_LOG")
    if not path:
        return
    rec = {"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], "what": what,
           "max_err_over_bound": float(ratio), "elements": int(n), "over_bound": int(over)}
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def _exponent_field(codes, fmt):
    """Unbiased exponent of each FP8 code's exponent field (subnormals and zero
    at the minimum normal exponent)."""
    c = codes.astype(np.int64) & 0x7F
    if fmt == 0:
        e = c >> 3
        return np.where(e > 0, e - 7, -6)
    e = c >> 2
    return np.where(e > 0, e - 15, -14)


def mfma_alignment_bound(a, sa, a_fmt, b_nk, sb_nk, b_fmt, b_scale):
    """Per-element error bound of the FP8 matrix cores for adversarial operands.

    Measured on gfx950 (every FP8 MFMA form): the products of each run of 8
    consecutive k are aligned to the run's largest exponent sum
    E = max(e_a + e_b), bits below 2^(E-13) are truncated toward zero, and the
    runs' sums accumulate in fp32.  Each of the <= 8 products of a run
    therefore loses less than 2^(E-13), times the run's scale.  For operands
    whose products span a narrow range this is far below 2^-12 * sum|a*b|; for
    uniformly random codes (products spanning ~50 binades) an element can
    exceed that by a few percent, rarely.  a: [M][K] codes, b_nk: [N][K] codes,
    sb_nk: per-row [N][K/128] (b_scale ROW128) or per-block [ceil(N/128)][K/128]."""
    M, K = a.shape
    N = b_nk.shape[0]
    ea = _exponent_field(a, a_fmt)
    eb = _exponent_field(b_nk, b_fmt)
    sbr = _b_row_scales(sb_nk, b_scale, N)
    bound = np.zeros((M, N))
    for g in range(K // 8):
        k0 = 8 * g
        E = np.max(ea[:, None, k0:k0 + 8] + eb[None, :, k0:k0 + 8], axis=2)
        sc = (sa[:, k0 // 128].astype(np.int64)[:, None] - 127) + (sbr[:, k0 // 128].astype(np.int64)[None, :] - 127)
        bound += 8.0 * np.exp2((E - 13 + sc).astype(np.float64))
    return bound


def _b_row_scales(sb_nk, b_scale, N):
    return sb_nk if b_scale == mx.SCALE_ROW128 else np.repeat(sb_nk, 128, axis=0)[:N]


def mfma_alignment_bound_at(a, sa, a_fmt, b_nk, sb_nk, b_fmt, b_scale, ii, jj):
    """The same bound for the listed output elements (ii[p], jj[p])."""
    K = a.shape[1]
    N = b_nk.shape[0]
    sbr = _b_row_scales(sb_nk, b_scale, N)
    E = (_exponent_field(a[ii], a_fmt) + _exponent_field(b_nk[jj], b_fmt)).reshape(len(ii), K // 8, 8).max(axis=2)
    sc = (np.repeat(sa[ii].astype(np.int64), 16, axis=1) - 127) + (np.repeat(sbr[jj].astype(np.int64), 16, axis=1) - 127)
    return (8.0 * np.exp2((E - 13 + sc).astype(np.float64))).sum(axis=1)


def mx_alignment_bound(a, sa, a_fmt, b_nk, sb, b_fmt):
    """The matrix cores' alignment bound (see mfma_alignment_bound) for MX
    operands: scales [M][K/32] and [N][K/32], one per 32-wide K chunk."""
    M, K = a.shape
    N = b_nk.shape[0]
    ea = _exponent_field(a, a_fmt)
    eb = _exponent_field(b_nk, b_fmt)
    bound = np.zeros((M, N))
    for g in range(K // 8):
        k0 = 8 * g
        E = np.max(ea[:, None, k0:k0 + 8] + eb[None, :, k0:k0 + 8], axis=2)
        sc = (sa[:, k0 // 32].astype(np.int64)[:, None] - 127) + (sb[:, k0 // 32].astype(np.int64)[None, :] - 127)
        bound += 8.0 * np.exp2((E - 13 + sc).astype(np.float64))
    return bound


def mx_alignment_bound_at(a, sa, a_fmt, b_nk, sb, b_fmt, ii, jj):
    """mx_alignment_bound for the listed output elements (ii[p], jj[p])."""
    K = a.shape[1]
    E = (_exponent_field(a[ii], a_fmt) + _exponent_field(b_nk[jj], b_fmt)).reshape(len(ii), K // 8, 8).max(axis=2)
    sc = (np.repeat(sa[ii].astype(np.int64), 4, axis=1) - 127) + (np.repeat(sb[jj].astype(np.int64), 4, axis=1) - 127)
    return (8.0 * np.exp2((E - 13 + sc).astype(np.float64))).sum(axis=1)


def assert_gemm_close(y_gpu, y_ref, t_ref, bf16_out, what="", extra_rel=0.0, hw_bound=None, max_over_plain=0):
    """|y_gpu - y| <= 2^-12 * sum|a*b| (+ one bf16 rounding for bf16 output), element
    by element; every output must be finite.

    Adversarial random-code tests pass hw_bound, the matrix cores' own alignment
    bound (mfma_alignment_bound): then at most max_over_plain elements may exceed the
    plain bound, and those must stay within hw_bound.  The largest err / plain bound
    and the count above it are recorded (record_ratio)."""
    y_gpu = np.asarray(y_gpu)
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    tol = gemm_tolerance(y_ref, t_ref, bf16_out, extra_rel)
    assert np.isfinite(y_gpu).all(), what + ": non-finite output"
    ratio = err / np.maximum(tol, np.finfo(np.float64).tiny)
    ratio = np.where(err == 0, 0.0, ratio)
    over = err > tol
    record_ratio(what, ratio.max() if ratio.size else 0.0, ratio.size, int(over.sum()))
    if hw_bound is None or not over.any():
        bad = over
    else:
        assert int(over.sum()) <= max_over_plain, "%s: %d elements above the plain bound (cap %d); worst ratio %.4f" % (
            what, int(over.sum()), max_over_plain, float(ratio.max()))
        hb = hw_bound + 2.0 ** -20 * t_ref
        if bf16_out:
            hb = hb + 2.0 ** -8 * (np.abs(y_ref) + hb)
        tol = np.maximum(tol, hb)
        bad = err > tol
    assert not bad.any(), "%s: %d elements out of tolerance; worst err %.3e tol %.3e at %s" % (
        what, int(bad.sum()), float(err[bad].max()), float(tol[bad][np.argmax(err[bad])]),
        str(np.argwhere(bad)[0]))


def adversarial_cap(n):
    """Elements of an n-element random-code product allowed above the plain bound: one
    per 100,000 (at least one).  The matrix-core model puts the rate near one per
    400,000 for uniformly random codes."""
    return max(1, n // 100000)


def run_gemm(a, sa, a_fmt, b, sb, b_fmt, b_layout, b_scale, bf16_out):
    out = mx.block_scaled_gemm(dev_ld16(a), dev(sa), a_fmt, dev_ld16(b), dev(sb), b_fmt, b_layout, b_scale,
                               out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    torch.cuda.synchronize()
    return host(out)


def run_mx_gemm(a, sa, a_fmt, b, sb, b_fmt, bf16_out):
    out = mx.mx_scaled_gemm(dev_ld16(a), dev(sa), a_fmt, dev_ld16(b), dev(sb), b_fmt,
                            out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    torch.cuda.synchronize()
    return host(out)
