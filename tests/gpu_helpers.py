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


def _b_row_scales(sb_nk, b_scale, N):
    return sb_nk if b_scale == mx.SCALE_ROW128 else np.repeat(sb_nk, 128, axis=0)[:N]


def mfma_alignment_bound_at(a, sa, a_fmt, b_nk, sb_nk, b_fmt, b_scale, ii, jj):
    """Per-element error bound of the FP8 matrix cores for adversarial operands, at
    the listed output elements (ii[p], jj[p]).

    Measured on gfx950 (every FP8 MFMA form): the products of each run of 8
    consecutive k are aligned to the run's largest exponent sum
    E = max(e_a + e_b), bits below 2^(E-13) are truncated toward zero, and the
    runs' sums accumulate in fp32.  Each of the <= 8 products of a run therefore
    loses less than 2^(E-13), times the run's scale.  For operands whose products
    span a narrow range this is far below 2^-12 * sum|a*b|; for uniformly random
    codes (products spanning ~50 binades) an element can exceed that, rarely.
    a: [M][K] codes, b_nk: [N][K] codes, sb_nk: per-row [N][K/128] (b_scale
    ROW128) or per-block [ceil(N/128)][K/128]."""
    K = a.shape[1]
    N = b_nk.shape[0]
    sbr = _b_row_scales(sb_nk, b_scale, N)
    E = (_exponent_field(a[ii], a_fmt) + _exponent_field(b_nk[jj], b_fmt)).reshape(len(ii), K // 8, 8).max(axis=2)
    sc = (np.repeat(sa[ii].astype(np.int64), 16, axis=1) - 127) + (np.repeat(sbr[jj].astype(np.int64), 16, axis=1) - 127)
    return (8.0 * np.exp2((E - 13 + sc).astype(np.float64))).sum(axis=1)


def mx_alignment_bound_at(a, sa, a_fmt, b_nk, sb, b_fmt, ii, jj):
    """mfma_alignment_bound_at for MX operands (scales [M][K/32] and [N][K/32], one
    per 32-wide K chunk), at the listed output elements (ii[p], jj[p])."""
    K = a.shape[1]
    E = (_exponent_field(a[ii], a_fmt) + _exponent_field(b_nk[jj], b_fmt)).reshape(len(ii), K // 8, 8).max(axis=2)
    sc = (np.repeat(sa[ii].astype(np.int64), 4, axis=1) - 127) + (np.repeat(sb[jj].astype(np.int64), 4, axis=1) - 127)
    return (8.0 * np.exp2((E - 13 + sc).astype(np.float64))).sum(axis=1)


def assert_gemm_close(y_gpu, y_ref, t_ref, bf16_out, what="", extra_rel=0.0, hw_bound=None, max_over_plain=0):
    """|y_gpu - y| <= 2^-12 * sum|a*b| (+ one bf16 rounding for bf16 output), element
    by element; every output must be finite.

    Adversarial random-code tests pass hw_bound, a function of the index arrays of
    np.nonzero that returns the matrix cores' own alignment bound at those elements
    (alignment_bound_fn): then at most max_over_plain elements may exceed the plain
    bound, and those must stay within it.  The largest err / plain bound and the count
    above it are recorded (record_ratio)."""
    y_gpu = np.asarray(y_gpu)
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    tol = gemm_tolerance(y_ref, t_ref, bf16_out, extra_rel)
    assert np.isfinite(y_gpu).all(), what + ": non-finite output"
    ratio = err / np.maximum(tol, np.finfo(np.float64).tiny)
    ratio = np.where(err == 0, 0.0, ratio)
    over = err > tol
    n_over = int(over.sum())
    record_ratio(what, ratio.max() if ratio.size else 0.0, ratio.size, n_over)
    if n_over and hw_bound is not None:
        assert n_over <= max_over_plain, "%s: %d elements above the plain bound (cap %d); worst ratio %.4f" % (
            what, n_over, max_over_plain, float(ratio.max()))
        idx = np.nonzero(over)
        hb = np.asarray(hw_bound(idx), dtype=np.float64) + 2.0 ** -20 * t_ref[idx]
        if bf16_out:
            hb = hb + 2.0 ** -8 * (np.abs(y_ref[idx]) + hb)
        bad_hw = err[idx] > np.maximum(tol[idx], hb)
        assert not bad_hw.any(), "%s: %d elements above the alignment bound; first at %s (err %.3e bound %.3e)" % (
            what, int(bad_hw.sum()), str([int(i[np.argmax(bad_hw)]) for i in idx]),
            float(err[idx][np.argmax(bad_hw)]), float(hb[np.argmax(bad_hw)]))
        return
    assert not over.any(), "%s: %d elements out of tolerance; worst err %.3e tol %.3e at %s" % (
        what, n_over, float(err[over].max()), float(tol[over][np.argmax(err[over])]),
        str(np.argwhere(over)[0]))


def alignment_bound_fn(a, sa, a_fmt, b_nk, sb, b_fmt, b_scale=None, mx_scales=False, ii=None, jj=None):
    """hw_bound for assert_gemm_close: the alignment bound at the requested elements
    of the product of a [M][K] and b_nk [N][K] (block scales per b_scale, or MX scales
    [rows][K/32]).  With ii, jj, the compared array is the 1-D sample y[ii, jj]."""
    def fn(idx):
        if ii is not None:
            r, c = ii[idx[0]], jj[idx[0]]
        else:
            r, c = idx
        if mx_scales:
            return mx_alignment_bound_at(a, sa, a_fmt, b_nk, sb, b_fmt, r, c)
        return mfma_alignment_bound_at(a, sa, a_fmt, b_nk, sb, b_fmt, b_scale, r, c)
    return fn


def adversarial_cap(n):
    """Elements of an n-element product of uniformly random codes allowed above the
    plain bound (each still within the alignment bound): one per 10,000, at least one.
    A CPU model of the matrix cores' truncation puts the rate near one per 400,000 with
    one scale per 128 k and a few per 100,000 with one scale per 32 k (fewer runs
    share the dominant scale, so less of the truncation cancels)."""
    return max(1, n // 10000)


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
