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
#
# The C entry points take raw pointers and cannot see a tensor's extent, so
# the tensor conveniences below check every tensor before passing its
# pointer: dtype, the exact shape the header documents for it, unit column
# stride (dense for scale, count and bitwidth arrays), and that all tensors
# live on the current CUDA device, whose current stream (or the given one)
# the work goes to.  A mismatch raises ValueError before any call.

def _torch():
    import torch
    return torch


def _check(status, where):
    if status != 0:
        raise MxFp8Error(status, where)


def _require(cond, msg, *args):
    """Raise ValueError(msg % args) unless cond; the message is formatted only then."""
    if not cond:
        raise ValueError(msg % args if args else msg)


_DTYPES = {}


def _code_dtypes():
    d = _DTYPES.get("codes")
    if d is None:
        torch = _torch()
        d = _DTYPES["codes"] = tuple(x for x in (torch.uint8, getattr(torch, "float8_e4m3fn", None),
                                                 getattr(torch, "float8_e5m2", None)) if x is not None)
    return d


def _scale_dtypes():
    d = _DTYPES.get("scales")
    if d is None:
        torch = _torch()
        d = _DTYPES["scales"] = tuple(x for x in (torch.uint8, getattr(torch, "float8_e8m0fnu", None))
                                      if x is not None)
    return d


def _is_tensor(t):
    return isinstance(t, _torch().Tensor)


def _matrix(t, name, dtypes, shape):
    """A 2-D tensor of one of `dtypes`, of exactly `shape`, with unit column stride
    (rows may be padded: the row stride is passed as the leading dimension)."""
    _require(_is_tensor(t), "%s must be a torch tensor", name)
    sh = t.shape
    _require(len(sh) == 2, "%s must be 2-D, got %d-D", name, len(sh))
    if t.dtype not in dtypes:
        _require(False, "%s must have dtype %s, got %s", name, " or ".join(str(d) for d in dtypes), t.dtype)
    _require(sh[0] == shape[0] and sh[1] == shape[1], "%s must have shape %s, got %s", name, tuple(shape),
             tuple(sh))
    st = t.stride()
    _require(sh[1] <= 1 or st[1] == 1, "%s must have unit column stride", name)
    _require(sh[0] <= 1 or st[0] >= sh[1], "%s rows must not overlap", name)


def _dense(t, name, dtypes, shape):
    """A contiguous tensor of one of `dtypes` and exactly `shape` (scale, count and
    bitwidth arrays carry no leading dimension)."""
    _matrix(t, name, dtypes, shape)
    _require(t.is_contiguous(), "%s must be contiguous (dense %s)", name, tuple(shape))


def _device_of(named):
    """All tensors on one CUDA device, which must be the current device; returns
    its index.  (Integer device ids and the raw stream handle below keep the
    per-call cost of these checks to a few microseconds.)"""
    torch = _torch()
    dev = None
    for name, t in named:
        _require(t.is_cuda, "%s must be a CUDA tensor, got device %s", name, t.device)
        i = t.get_device()
        if dev is None:
            dev = i
        _require(i == dev, "%s is on cuda:%d but %s is on cuda:%d", name, i, named[0][0], dev)
    cur = torch.cuda.current_device()
    _require(dev == cur, "tensors are on cuda:%d but the current device is cuda:%d", dev, cur)
    return dev


def _stream(stream, dev):
    """The HIP stream handle for device index dev: the given torch stream (which
    must belong to dev), else dev's current stream."""
    torch = _torch()
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        return raw(dev) if raw is not None else torch.cuda.current_stream(dev).cuda_stream
    _require(stream.device.index == dev, "stream is on %s but the tensors are on cuda:%d", stream.device, dev)
    return stream.cuda_stream


def _in_dtype(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError("input must be float32 or bfloat16, got %s" % t.dtype)


def _input(x, name):
    """A float32 / bfloat16 2-D input with unit column stride; returns (rows, cols)."""
    torch = _torch()
    _require(_is_tensor(x) and x.dim() == 2, "%s must be a 2-D torch tensor", name)
    _matrix(x, name, (torch.float32, torch.bfloat16), tuple(x.shape))
    return x.shape


def _ld(t):
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _pad16(n):
    return (n + 15) // 16 * 16


def _cdiv(a, b):
    return (a + b - 1) // b


def _codes(rows, cols, device):
    """Uninitialized [rows][cols] uint8 view with a 16-element-aligned row pitch."""
    torch = _torch()
    buf = torch.empty((rows, _pad16(max(cols, 1))), dtype=torch.uint8, device=device)
    return buf[:, :cols]


def _check_out(out, out_dtype, M, N):
    """The GEMM output, if given: [M][N], float32 or bfloat16; otherwise out_dtype."""
    torch = _torch()
    if out is None:
        _require(out_dtype in (None, torch.float32, torch.bfloat16),
                 "out_dtype must be torch.float32 or torch.bfloat16, got %s", out_dtype)
    else:
        _matrix(out, "out", (torch.float32, torch.bfloat16), (M, N))


def _out_matrix(out, out_dtype, M, N, device):
    """`out` (already checked), or a new [M][N] output with a 16-element row pitch."""
    torch = _torch()
    if out is not None:
        return out
    dt = torch.bfloat16 if out_dtype == torch.bfloat16 else torch.float32
    buf = torch.empty((M, _pad16(max(N, 1))), dtype=dt, device=device)
    return buf[:, :N]


def quantize_token(x, fmt=E4M3, axis=ROW, stream=None):
    """Token-wise 1x128 quantization.  ROW: (q [rows][cols], scales [rows][ceil(cols/128)]).
    COL_T: (qt [cols][rows], scales [cols][ceil(rows/128)])."""
    torch = _torch()
    rows, cols = _input(x, "x")
    dev = _device_of([("x", x)])
    if axis == ROW:
        q = _codes(rows, cols, dev)
        s = torch.empty((rows, _cdiv(cols, 128)), dtype=torch.uint8, device=dev)
    else:
        q = _codes(cols, rows, dev)
        s = torch.empty((cols, _cdiv(rows, 128)), dtype=torch.uint8, device=dev)
    st = fp8_quantize_token(x.data_ptr(), _in_dtype(x), rows, cols, _ld(x), axis, fmt, q.data_ptr(), _ld(q),
                            s.data_ptr(), _stream(stream, dev))
    _check(st, "fp8_quantize_token")
    return q, s


def quantize_block(w, fmt=E4M3, stream=None):
    """128x128 block quantization: (q [rows][cols], scales [ceil(rows/128)][ceil(cols/128)])."""
    torch = _torch()
    rows, cols = _input(w, "w")
    dev = _device_of([("w", w)])
    q = _codes(rows, cols, dev)
    s = torch.empty((_cdiv(rows, 128), _cdiv(cols, 128)), dtype=torch.uint8, device=dev)
    st = fp8_quantize_block(w.data_ptr(), _in_dtype(w), rows, cols, _ld(w), fmt, q.data_ptr(), _ld(q),
                            s.data_ptr(), _stream(stream, dev))
    _check(st, "fp8_quantize_block")
    return q, s


def quantize_token_f32s(x, fmt=E4M3, axis=ROW, stream=None):
    """quantize_token with fp32 scales (float32 tensors in the same layouts)."""
    torch = _torch()
    rows, cols = _input(x, "x")
    dev = _device_of([("x", x)])
    if axis == ROW:
        q = _codes(rows, cols, dev)
        s = torch.empty((rows, _cdiv(cols, 128)), dtype=torch.float32, device=dev)
    else:
        q = _codes(cols, rows, dev)
        s = torch.empty((cols, _cdiv(rows, 128)), dtype=torch.float32, device=dev)
    st = fp8_quantize_token_f32s(x.data_ptr(), _in_dtype(x), rows, cols, _ld(x), axis, fmt, q.data_ptr(), _ld(q),
                                 s.data_ptr(), _stream(stream, dev))
    _check(st, "fp8_quantize_token_f32s")
    return q, s


def quantize_block_f32s(w, fmt=E4M3, stream=None):
    """quantize_block with fp32 scales."""
    torch = _torch()
    rows, cols = _input(w, "w")
    dev = _device_of([("w", w)])
    q = _codes(rows, cols, dev)
    s = torch.empty((_cdiv(rows, 128), _cdiv(cols, 128)), dtype=torch.float32, device=dev)
    st = fp8_quantize_block_f32s(w.data_ptr(), _in_dtype(w), rows, cols, _ld(w), fmt, q.data_ptr(), _ld(q),
                                 s.data_ptr(), _stream(stream, dev))
    _check(st, "fp8_quantize_block_f32s")
    return q, s


def quantize_token_dual(x, fmt=E4M3, stream=None):
    """Both token orientations from one read: (q, scales) as quantize_token ROW and
    (qt, scales_t) as quantize_token COL_T."""
    torch = _torch()
    rows, cols = _input(x, "x")
    dev = _device_of([("x", x)])
    q = _codes(rows, cols, dev)
    s = torch.empty((rows, _cdiv(cols, 128)), dtype=torch.uint8, device=dev)
    qt = _codes(cols, rows, dev)
    st = torch.empty((cols, _cdiv(rows, 128)), dtype=torch.uint8, device=dev)
    r = fp8_quantize_token_dual(x.data_ptr(), _in_dtype(x), rows, cols, _ld(x), fmt, q.data_ptr(), _ld(q),
                                s.data_ptr(), qt.data_ptr(), _ld(qt), st.data_ptr(), _stream(stream, dev))
    _check(r, "fp8_quantize_token_dual")
    return q, s, qt, st


def quantize_block_dual(w, fmt=E4M3, stream=None):
    """128x128 block quantization with the transposed codes: (q, scales, qt, scales_t)."""
    torch = _torch()
    rows, cols = _input(w, "w")
    dev = _device_of([("w", w)])
    q = _codes(rows, cols, dev)
    s = torch.empty((_cdiv(rows, 128), _cdiv(cols, 128)), dtype=torch.uint8, device=dev)
    qt = _codes(cols, rows, dev)
    st = torch.empty((_cdiv(cols, 128), _cdiv(rows, 128)), dtype=torch.uint8, device=dev)
    r = fp8_quantize_block_dual(w.data_ptr(), _in_dtype(w), rows, cols, _ld(w), fmt, q.data_ptr(), _ld(q),
                                s.data_ptr(), qt.data_ptr(), _ld(qt), st.data_ptr(), _stream(stream, dev))
    _check(r, "fp8_quantize_block_dual")
    return q, s, qt, st


def quantize_mx(x, fmt=E4M3, rule=RULE_FLOOR, counts=True, stream=None):
    """MX 32-element quantization: (q, scales [rows][cols/32], counts [rows][cols/32] or None)."""
    torch = _torch()
    rows, cols = _input(x, "x")
    _require(cols % 32 == 0, "x must have a multiple of 32 columns, got %d", cols)
    dev = _device_of([("x", x)])
    q = _codes(rows, cols, dev)
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    c = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev) if counts else None
    st = mx_quantize(x.data_ptr(), _in_dtype(x), rows, cols, _ld(x), fmt, rule, q.data_ptr(), _ld(q),
                     s.data_ptr(), c.data_ptr() if counts else None, _stream(stream, dev))
    _check(st, "mx_quantize")
    return q, s, c


def _gemm_operands(a, a_scales, b, b_scales, b_layout, b_scale_mode, scale_dtypes, what):
    """Checks the operands of the block-scaled GEMMs; returns (M, N, K)."""
    _require(b_layout in (B_NK, B_KN), "b_layout must be B_NK or B_KN, got %r", b_layout)
    _require(b_scale_mode in (SCALE_BLOCK128, SCALE_ROW128),
             "b_scale_mode must be SCALE_BLOCK128 or SCALE_ROW128, got %r", b_scale_mode)
    _require(not (b_layout == B_KN and b_scale_mode == SCALE_ROW128), "%s: per-row B scales need B stored [N][K]",
             what)
    _require(_is_tensor(a) and a.dim() == 2, "a must be a 2-D torch tensor")
    _require(_is_tensor(b) and b.dim() == 2, "b must be a 2-D torch tensor")
    M, K = a.shape
    N = b.shape[0] if b_layout == B_NK else b.shape[1]
    _require(K % 128 == 0, "%s: K must be a multiple of 128, got %d", what, K)
    codes = _code_dtypes()
    _matrix(a, "a", codes, (M, K))
    _matrix(b, "b", codes, (N, K) if b_layout == B_NK else (K, N))
    _dense(a_scales, "a_scales", scale_dtypes, (M, K // 128))
    if b_scale_mode == SCALE_ROW128:
        sb_shape = (N, K // 128)
    elif b_layout == B_NK:
        sb_shape = (_cdiv(N, 128), K // 128)
    else:
        sb_shape = (K // 128, _cdiv(N, 128))
    _dense(b_scales, "b_scales", scale_dtypes, sb_shape)
    return M, N, K


def block_scaled_gemm(a, a_scales, a_fmt, b, b_scales, b_fmt, b_layout=B_NK, b_scale_mode=SCALE_BLOCK128,
                      out_dtype=None, out=None, stream=None):
    """C = A * B over block-scaled FP8 codes (uint8 or float8 tensors) with E8M0 scale
    bytes (uint8 or float8_e8m0fnu), fp32 accumulation.  a [M][K] with a_scales
    [M][K/128]; b [N][K] (B_NK) or [K][N] (B_KN) with b_scales [ceil(N/128)][K/128]
    (B_NK, SCALE_BLOCK128), [K/128][ceil(N/128)] (B_KN) or [N][K/128] (SCALE_ROW128)."""
    M, N, K = _gemm_operands(a, a_scales, b, b_scales, b_layout, b_scale_mode, _scale_dtypes(),
                             "block_scaled_gemm")
    _check_out(out, out_dtype, M, N)
    dev = _device_of([("a", a), ("a_scales", a_scales), ("b", b), ("b_scales", b_scales)]
                     + ([("out", out)] if out is not None else []))
    out = _out_matrix(out, out_dtype, M, N, dev)
    c_dtype = F32 if out.dtype == _torch().float32 else BF16
    st = fp8_block_scaled_gemm(M, N, K, a.data_ptr(), _ld(a), a_fmt, a_scales.data_ptr(), b.data_ptr(), _ld(b),
                               b_fmt, b_layout, b_scales.data_ptr(), b_scale_mode, out.data_ptr(), _ld(out),
                               c_dtype, _stream(stream, dev))
    _check(st, "fp8_block_scaled_gemm")
    return out


def mx_scaled_gemm(a, a_scales, a_fmt, b, b_scales, b_fmt, out_dtype=None, out=None, stream=None):
    """C = A * B^T over MX codes: a [M][K], b [N][K], scales [M][K/32] and [N][K/32]
    (quantize_mx's layout; uint8 or float8_e8m0fnu)."""
    _require(_is_tensor(a) and a.dim() == 2, "a must be a 2-D torch tensor")
    _require(_is_tensor(b) and b.dim() == 2, "b must be a 2-D torch tensor")
    M, K = a.shape
    N = b.shape[0]
    _require(K % 128 == 0, "mx_scaled_gemm: K must be a multiple of 128, got %d", K)
    codes = _code_dtypes()
    _matrix(a, "a", codes, (M, K))
    _matrix(b, "b", codes, (N, K))
    _dense(a_scales, "a_scales", _scale_dtypes(), (M, K // 32))
    _dense(b_scales, "b_scales", _scale_dtypes(), (N, K // 32))
    _check_out(out, out_dtype, M, N)
    dev = _device_of([("a", a), ("a_scales", a_scales), ("b", b), ("b_scales", b_scales)]
                     + ([("out", out)] if out is not None else []))
    out = _out_matrix(out, out_dtype, M, N, dev)
    c_dtype = F32 if out.dtype == _torch().float32 else BF16
    st = mx_gemm(M, N, K, a.data_ptr(), _ld(a), a_fmt, a_scales.data_ptr(), b.data_ptr(), _ld(b), b_fmt,
                 b_scales.data_ptr(), out.data_ptr(), _ld(out), c_dtype, _stream(stream, dev))
    _check(st, "mx_gemm")
    return out


def gemm_f32s(a, a_scales, a_fmt, b, b_scales, b_fmt, b_layout=B_NK, b_scale_mode=SCALE_BLOCK128,
              out_dtype=None, out=None, stream=None):
    """block_scaled_gemm over operands with fp32 scales (float32 tensors, same shapes)."""
    M, N, K = _gemm_operands(a, a_scales, b, b_scales, b_layout, b_scale_mode, (_torch().float32,), "gemm_f32s")
    _check_out(out, out_dtype, M, N)
    dev = _device_of([("a", a), ("a_scales", a_scales), ("b", b), ("b_scales", b_scales)]
                     + ([("out", out)] if out is not None else []))
    out = _out_matrix(out, out_dtype, M, N, dev)
    c_dtype = F32 if out.dtype == _torch().float32 else BF16
    st = fp8_gemm_f32s(M, N, K, a.data_ptr(), _ld(a), a_fmt, a_scales.data_ptr(), b.data_ptr(), _ld(b), b_fmt,
                       b_layout, b_scales.data_ptr(), b_scale_mode, out.data_ptr(), _ld(out), c_dtype,
                       _stream(stream, dev))
    _check(st, "fp8_gemm_f32s")
    return out


def gaussws(w, bitwidths, seed, stream_id=0, out=None, stream=None):
    """GaussWS sampled weight (bf16 tensor) of w with int8 bitwidths per 32x32 block
    ([ceil(rows/32)][ceil(cols/32)], contiguous)."""
    torch = _torch()
    rows, cols = _input(w, "w")
    _dense(bitwidths, "bitwidths", (torch.int8,), (_cdiv(rows, 32), _cdiv(cols, 32)))
    if out is not None:
        _matrix(out, "out", (torch.bfloat16,), (rows, cols))
    dev = _device_of([("w", w), ("bitwidths", bitwidths)] + ([("out", out)] if out is not None else []))
    if out is None:
        buf = torch.empty((rows, _pad16(max(cols, 1))), dtype=torch.bfloat16, device=dev)
        out = buf[:, :cols]
    st = gaussws_sample(w.data_ptr(), _in_dtype(w), rows, cols, _ld(w), bitwidths.data_ptr(), seed, stream_id,
                        out.data_ptr(), _ld(out), _stream(stream, dev))
    _check(st, "gaussws_sample")
    return out
