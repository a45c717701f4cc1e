"""mx_block_scaled_x128_amd -- MI355X (gfx950) FP8 quantization and block-scaled GEMM.

Thin Python binding over the C ABI of ``libmxfp8.so`` (include/mxfp8.h).  It
marshals arguments only: every step of quantization and of the GEMM runs in
the HIP kernels of the library.  torch supplies device memory and the current
stream; nothing here computes.  If the library has not been built, every
entry point raises -- there is no fallback path.

Low-level entry points carry the C names and signatures (pointers as ints):
  fp8_quantize_token, fp8_quantize_block, fp8_quantize_token_dual,
  fp8_quantize_block_dual, fp8_quantize_token_f32s, fp8_quantize_block_f32s,
  mx_quantize, fp8_block_scaled_gemm, fp8_gemm_f32s, mx_gemm, gaussws_sample,
  mxfp8_status_string, mxfp8_version.
Tensor conveniences allocate outputs with torch and call them:
  quantize_token, quantize_block, quantize_token_dual, quantize_block_dual,
  quantize_token_f32s, quantize_block_f32s, quantize_mx, block_scaled_gemm,
  gemm_f32s, mx_scaled_gemm, gaussws.
"""
import ctypes
import os
import threading

__all__ = [
    "E4M3", "E5M2", "F32", "BF16", "ROW", "COL_T", "RULE_CEIL", "RULE_FLOOR", "B_NK", "B_KN",
    "SCALE_BLOCK128", "SCALE_ROW128", "MxFp8Error", "library_path", "load_library",
    "fp8_quantize_token", "fp8_quantize_block", "fp8_quantize_token_dual", "fp8_quantize_block_dual",
    "fp8_quantize_token_f32s", "fp8_quantize_block_f32s", "mx_quantize", "fp8_block_scaled_gemm",
    "fp8_gemm_f32s", "mx_gemm", "gaussws_sample", "mxfp8_status_string", "mxfp8_version",
    "quantize_token", "quantize_block", "quantize_token_dual", "quantize_block_dual",
    "quantize_token_f32s", "quantize_block_f32s", "quantize_mx", "block_scaled_gemm", "gemm_f32s",
    "mx_scaled_gemm", "gaussws",
]

# enum values of include/mxfp8.h
E4M3, E5M2 = 0, 1
F32, BF16 = 0, 1
ROW, COL_T = 0, 1
RULE_CEIL, RULE_FLOOR = 0, 1
B_NK, B_KN = 0, 1
SCALE_BLOCK128, SCALE_ROW128 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxfp8.so")
_lib = None
_lock = threading.Lock()


class MxFp8Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s failed: status %d (%s)" % (where, status, mxfp8_status_string(status)))


def library_path():
    return _LIB_PATH


def load_library():
    """Load libmxfp8.so (built in-tree by mx_block_scaled_x128_amd.build); raise if absent."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libmxfp8.so is not built (%s); run python -m mx_block_scaled_x128_amd.build"
                              % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.fp8_quantize_token.argtypes = [P, I, I64, I64, I64, I, I, P, I64, P, P]
        lib.fp8_quantize_token.restype = I
        lib.fp8_quantize_block.argtypes = [P, I, I64, I64, I64, I, P, I64, P, P]
        lib.fp8_quantize_block.restype = I
        lib.fp8_quantize_token_dual.argtypes = [P, I, I64, I64, I64, I, P, I64, P, P, I64, P, P]
        lib.fp8_quantize_token_dual.restype = I
        lib.fp8_quantize_block_dual.argtypes = [P, I, I64, I64, I64, I, P, I64, P, P, I64, P, P]
        lib.fp8_quantize_block_dual.restype = I
        lib.fp8_quantize_token_f32s.argtypes = [P, I, I64, I64, I64, I, I, P, I64, P, P]
        lib.fp8_quantize_token_f32s.restype = I
        lib.fp8_quantize_block_f32s.argtypes = [P, I, I64, I64, I64, I, P, I64, P, P]
        lib.fp8_quantize_block_f32s.restype = I
        lib.mx_quantize.argtypes = [P, I, I64, I64, I64, I, I, P, I64, P, P, P]
        lib.mx_quantize.restype = I
        lib.fp8_block_scaled_gemm.argtypes = [I64, I64, I64, P, I64, I, P, P, I64, I, I, P, I, P, I64, I, P]
        lib.fp8_block_scaled_gemm.restype = I
        lib.fp8_gemm_f32s.argtypes = [I64, I64, I64, P, I64, I, P, P, I64, I, I, P, I, P, I64, I, P]
        lib.fp8_gemm_f32s.restype = I
        lib.mx_gemm.argtypes = [I64, I64, I64, P, I64, I, P, P, I64, I, P, P, I64, I, P]
        lib.mx_gemm.restype = I
        lib.gaussws_sample.argtypes = [P, I, I64, I64, I64, P, ctypes.c_uint64, ctypes.c_uint64, P, I64, P]
        lib.gaussws_sample.restype = I
        lib.mxfp8_status_string.argtypes = [I]
        lib.mxfp8_status_string.restype = ctypes.c_char_p
        lib.mxfp8_version.argtypes = []
        lib.mxfp8_version.restype = I
        _lib = lib
        return lib


# --------------------------------------------------------------- C-named entry points

def fp8_quantize_token(x, x_dtype, rows, cols, ldx, axis, fmt, q, ldq, scales, stream):
    return load_library().fp8_quantize_token(x, x_dtype, rows, cols, ldx, axis, fmt, q, ldq, scales, stream)


def fp8_quantize_block(w, w_dtype, rows, cols, ldw, fmt, q, ldq, scales, stream):
    return load_library().fp8_quantize_block(w, w_dtype, rows, cols, ldw, fmt, q, ldq, scales, stream)


def fp8_quantize_token_f32s(x, x_dtype, rows, cols, ldx, axis, fmt, q, ldq, scales, stream):
    return load_library().fp8_quantize_token_f32s(x, x_dtype, rows, cols, ldx, axis, fmt, q, ldq, scales, stream)


def fp8_quantize_block_f32s(w, w_dtype, rows, cols, ldw, fmt, q, ldq, scales, stream):
    return load_library().fp8_quantize_block_f32s(w, w_dtype, rows, cols, ldw, fmt, q, ldq, scales, stream)


def fp8_quantize_token_dual(x, x_dtype, rows, cols, ldx, fmt, q, ldq, scales, qt, ldqt, scales_t, stream):
    return load_library().fp8_quantize_token_dual(x, x_dtype, rows, cols, ldx, fmt, q, ldq, scales, qt, ldqt,
                                                  scales_t, stream)


def fp8_quantize_block_dual(w, w_dtype, rows, cols, ldw, fmt, q, ldq, scales, qt, ldqt, scales_t, stream):
    return load_library().fp8_quantize_block_dual(w, w_dtype, rows, cols, ldw, fmt, q, ldq, scales, qt, ldqt,
                                                  scales_t, stream)


def mx_quantize(x, x_dtype, rows, cols, ldx, fmt, rule, q, ldq, scales, clamp_counts, stream):
    return load_library().mx_quantize(x, x_dtype, rows, cols, ldx, fmt, rule, q, ldq, scales, clamp_counts,
                                      stream)


def fp8_block_scaled_gemm(M, N, K, a, lda, a_fmt, a_scales, b, ldb, b_fmt, b_layout, b_scales, b_scale_mode,
                          c, ldc, c_dtype, stream):
    return load_library().fp8_block_scaled_gemm(M, N, K, a, lda, a_fmt, a_scales, b, ldb, b_fmt, b_layout,
                                                 b_scales, b_scale_mode, c, ldc, c_dtype, stream)


def fp8_gemm_f32s(M, N, K, a, lda, a_fmt, a_scales, b, ldb, b_fmt, b_layout, b_scales, b_scale_mode, c, ldc,
                  c_dtype, stream):
    return load_library().fp8_gemm_f32s(M, N, K, a, lda, a_fmt, a_scales, b, ldb, b_fmt, b_layout, b_scales,
                                        b_scale_mode, c, ldc, c_dtype, stream)


def mx_gemm(M, N, K, a, lda, a_fmt, a_scales, b, ldb, b_fmt, b_scales, c, ldc, c_dtype, stream):
    return load_library().mx_gemm(M, N, K, a, lda, a_fmt, a_scales, b, ldb, b_fmt, b_scales, c, ldc, c_dtype,
                                  stream)


def gaussws_sample(w, w_dtype, rows, cols, ldw, bitwidths, seed, stream_id, w_hat, ldo, stream):
    return load_library().gaussws_sample(w, w_dtype, rows, cols, ldw, bitwidths, seed, stream_id, w_hat, ldo,
                                         stream)


def mxfp8_status_string(status):
    return load_library().mxfp8_status_string(status).decode()


def mxfp8_version():
    return load_library().mxfp8_version()


# ------------------------------------------------------------------ tensor helpers

def _torch():
    import torch
    return torch


def _check(status, where):
    if status != 0:
        raise MxFp8Error(status, where)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _in_dtype(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("input must be float32 or bfloat16, got %s" % t.dtype)


def _ld(t):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


def _pad16(n):
    return (n + 15) // 16 * 16


def _codes(rows, cols, device):
    """Uninitialized [rows][cols] uint8 view with a 16-element-aligned row pitch."""
    torch = _torch()
    buf = torch.empty((rows, _pad16(max(cols, 1))), dtype=torch.uint8, device=device)
    return buf[:, :cols]


def quantize_token(x, fmt=E4M3, axis=ROW, stream=None):
    """Token-wise 1x128 quantization.  ROW: (q [rows][cols], scales [rows][ceil(cols/128)]).
    COL_T: (qt [cols][rows], scales [cols][ceil(rows/128)])."""
    torch = _torch()
    rows, cols = x.shape
    if axis == ROW:
        q = _codes(rows, cols, x.device)
        s = torch.empty((rows, (cols + 127) // 128), dtype=torch.uint8, device=x.device)
    else:
        q = _codes(cols, rows, x.device)
        s = torch.empty((cols, (rows + 127) // 128), dtype=torch.uint8, device=x.device)
    st = fp8_quantize_token(x.data_ptr(), _in_dtype(x), rows, cols, _ld(x), axis, fmt, q.data_ptr(), _ld(q),
                            s.data_ptr(), _stream(stream))
    _check(st, "fp8_quantize_token")
    return q, s


def quantize_block(w, fmt=E4M3, stream=None):
    """128x128 block quantization: (q [rows][cols], scales [ceil(rows/128)][ceil(cols/128)])."""
    torch = _torch()
    rows, cols = w.shape
    q = _codes(rows, cols, w.device)
    s = torch.empty(((rows + 127) // 128, (cols + 127) // 128), dtype=torch.uint8, device=w.device)
    st = fp8_quantize_block(w.data_ptr(), _in_dtype(w), rows, cols, _ld(w), fmt, q.data_ptr(), _ld(q),
                            s.data_ptr(), _stream(stream))
    _check(st, "fp8_quantize_block")
    return q, s


def quantize_token_f32s(x, fmt=E4M3, axis=ROW, stream=None):
    """quantize_token with fp32 scales (float32 tensors in the same layouts)."""
    torch = _torch()
    rows, cols = x.shape
    if axis == ROW:
        q = _codes(rows, cols, x.device)
        s = torch.empty((rows, (cols + 127) // 128), dtype=torch.float32, device=x.device)
    else:
        q = _codes(cols, rows, x.device)
        s = torch.empty((cols, (rows + 127) // 128), dtype=torch.float32, device=x.device)
    st = fp8_quantize_token_f32s(x.data_ptr(), _in_dtype(x), rows, cols, _ld(x), axis, fmt, q.data_ptr(), _ld(q),
                                 s.data_ptr(), _stream(stream))
    _check(st, "fp8_quantize_token_f32s")
    return q, s


def quantize_block_f32s(w, fmt=E4M3, stream=None):
    """quantize_block with fp32 scales."""
    torch = _torch()
    rows, cols = w.shape
    q = _codes(rows, cols, w.device)
    s = torch.empty(((rows + 127) // 128, (cols + 127) // 128), dtype=torch.float32, device=w.device)
    st = fp8_quantize_block_f32s(w.data_ptr(), _in_dtype(w), rows, cols, _ld(w), fmt, q.data_ptr(), _ld(q),
                                 s.data_ptr(), _stream(stream))
    _check(st, "fp8_quantize_block_f32s")
    return q, s


def quantize_token_dual(x, fmt=E4M3, stream=None):
    """Both token orientations from one read: (q, scales) as quantize_token ROW and
    (qt, scales_t) as quantize_token COL_T."""
    torch = _torch()
    rows, cols = x.shape
    q = _codes(rows, cols, x.device)
    s = torch.empty((rows, (cols + 127) // 128), dtype=torch.uint8, device=x.device)
    qt = _codes(cols, rows, x.device)
    st = torch.empty((cols, (rows + 127) // 128), dtype=torch.uint8, device=x.device)
    r = fp8_quantize_token_dual(x.data_ptr(), _in_dtype(x), rows, cols, _ld(x), fmt, q.data_ptr(), _ld(q),
                                s.data_ptr(), qt.data_ptr(), _ld(qt), st.data_ptr(), _stream(stream))
    _check(r, "fp8_quantize_token_dual")
    return q, s, qt, st


def quantize_block_dual(w, fmt=E4M3, stream=None):
    """128x128 block quantization with the transposed codes: (q, scales, qt, scales_t)."""
    torch = _torch()
    rows, cols = w.shape
    q = _codes(rows, cols, w.device)
    s = torch.empty(((rows + 127) // 128, (cols + 127) // 128), dtype=torch.uint8, device=w.device)
    qt = _codes(cols, rows, w.device)
    st = torch.empty(((cols + 127) // 128, (rows + 127) // 128), dtype=torch.uint8, device=w.device)
    r = fp8_quantize_block_dual(w.data_ptr(), _in_dtype(w), rows, cols, _ld(w), fmt, q.data_ptr(), _ld(q),
                                s.data_ptr(), qt.data_ptr(), _ld(qt), st.data_ptr(), _stream(stream))
    _check(r, "fp8_quantize_block_dual")
    return q, s, qt, st


def quantize_mx(x, fmt=E4M3, rule=RULE_FLOOR, counts=True, stream=None):
    """MX 32-element quantization: (q, scales [rows][cols/32], counts [rows][cols/32] or None)."""
    torch = _torch()
    rows, cols = x.shape
    q = _codes(rows, cols, x.device)
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    c = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device) if counts else None
    st = mx_quantize(x.data_ptr(), _in_dtype(x), rows, cols, _ld(x), fmt, rule, q.data_ptr(), _ld(q),
                     s.data_ptr(), c.data_ptr() if counts else None, _stream(stream))
    _check(st, "mx_quantize")
    return q, s, c


def block_scaled_gemm(a, a_scales, a_fmt, b, b_scales, b_fmt, b_layout=B_NK, b_scale_mode=SCALE_BLOCK128,
                      out_dtype=None, out=None, stream=None):
    """C = A * B over block-scaled FP8 codes (uint8 tensors), fp32 accumulation."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[0] if b_layout == B_NK else b.shape[1]
    if out is None:
        dt = torch.float32 if out_dtype in (None, torch.float32) else torch.bfloat16
        buf = torch.empty((M, _pad16(max(N, 1))), dtype=dt, device=a.device)
        out = buf[:, :N]
    c_dtype = F32 if out.dtype == torch.float32 else BF16
    st = fp8_block_scaled_gemm(M, N, K, a.data_ptr(), _ld(a), a_fmt, a_scales.data_ptr(), b.data_ptr(), _ld(b),
                               b_fmt, b_layout, b_scales.data_ptr(), b_scale_mode, out.data_ptr(), _ld(out),
                               c_dtype, _stream(stream))
    _check(st, "fp8_block_scaled_gemm")
    return out


def mx_scaled_gemm(a, a_scales, a_fmt, b, b_scales, b_fmt, out_dtype=None, out=None, stream=None):
    """C = A * B^T over MX codes: a [M][K], b [N][K], scales [rows][K/32] (quantize_mx's layout)."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[0]
    if out is None:
        dt = torch.float32 if out_dtype in (None, torch.float32) else torch.bfloat16
        buf = torch.empty((M, _pad16(max(N, 1))), dtype=dt, device=a.device)
        out = buf[:, :N]
    c_dtype = F32 if out.dtype == torch.float32 else BF16
    st = mx_gemm(M, N, K, a.data_ptr(), _ld(a), a_fmt, a_scales.data_ptr(), b.data_ptr(), _ld(b), b_fmt,
                 b_scales.data_ptr(), out.data_ptr(), _ld(out), c_dtype, _stream(stream))
    _check(st, "mx_gemm")
    return out


def gemm_f32s(a, a_scales, a_fmt, b, b_scales, b_fmt, b_layout=B_NK, b_scale_mode=SCALE_BLOCK128,
              out_dtype=None, out=None, stream=None):
    """block_scaled_gemm over operands with fp32 (float32 tensor) scales."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[0] if b_layout == B_NK else b.shape[1]
    if out is None:
        dt = torch.float32 if out_dtype in (None, torch.float32) else torch.bfloat16
        buf = torch.empty((M, _pad16(max(N, 1))), dtype=dt, device=a.device)
        out = buf[:, :N]
    c_dtype = F32 if out.dtype == torch.float32 else BF16
    st = fp8_gemm_f32s(M, N, K, a.data_ptr(), _ld(a), a_fmt, a_scales.data_ptr(), b.data_ptr(), _ld(b), b_fmt,
                       b_layout, b_scales.data_ptr(), b_scale_mode, out.data_ptr(), _ld(out), c_dtype,
                       _stream(stream))
    _check(st, "fp8_gemm_f32s")
    return out


def gaussws(w, bitwidths, seed, stream_id=0, out=None, stream=None):
    """GaussWS sampled weight (bf16 tensor) of w with int8 bitwidths per 32x32 block."""
    torch = _torch()
    rows, cols = w.shape
    if out is None:
        buf = torch.empty((rows, _pad16(max(cols, 1))), dtype=torch.bfloat16, device=w.device)
        out = buf[:, :cols]
    st = gaussws_sample(w.data_ptr(), _in_dtype(w), rows, cols, _ld(w), bitwidths.data_ptr(), seed, stream_id,
                        out.data_ptr(), _ld(out), _stream(stream))
    _check(st, "gaussws_sample")
    return out
