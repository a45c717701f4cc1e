"""Helpers for the GPU parity tests: host <-> device marshalling and the
tolerances of the block-scaled GEMM."""
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


def gemm_tolerance(y_ref, t_ref, bf16_out):
    """Per-element bound: 2^-12 * sum|a*b| for fp32 output; one extra bf16 rounding
    (unit roundoff 2^-8 of a value within 2^-12 * t of y) for bf16 output."""
    tol = 2.0 ** -12 * t_ref
    if bf16_out:
        tol = tol + 2.0 ** -8 * (np.abs(y_ref) + 2.0 ** -12 * t_ref)
    return tol


def assert_gemm_close(y_gpu, y_ref, t_ref, bf16_out, what=""):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    tol = gemm_tolerance(y_ref, t_ref, bf16_out)
    bad = err > tol
    assert np.isfinite(y_gpu).all(), what + ": non-finite output"
    assert not bad.any(), "%s: %d elements out of tolerance; worst err %.3e tol %.3e at %s" % (
        what, int(bad.sum()), float(err[bad].max()), float(tol[bad][np.argmax(err[bad])]),
        str(np.argwhere(bad)[0]))


def run_gemm(a, sa, a_fmt, b, sb, b_fmt, b_layout, b_scale, bf16_out):
    out = mx.block_scaled_gemm(dev_ld16(a), dev(sa), a_fmt, dev_ld16(b), dev(sb), b_fmt, b_layout, b_scale,
                               out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    torch.cuda.synchronize()
    return host(out)
