"""CPU oracle for hybrid-granularity FP8 quantization and the block-scaled GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark import this package; the product library
never does.  The arithmetic lives in ``oracle.c`` (plain C, fp64, gcc -O2);
this module only marshals numpy arrays into it and, for speed on large
inputs, splits independent rows over host threads (each C call is
single-threaded; ctypes releases the GIL while it runs).

Integer conventions (this package's own):
  fmt 0 = E4M3, 1 = E5M2;  rule 0 = round-up scale, 1 = OCP floor scale;
  b_layout 0 = B stored [N][K], 1 = B stored [K][N];
  b_scale 0 = one scale per 128x128 tile of B's storage, 1 = per (n, K block).

Inputs: fp32 arrays (numpy float32) or bf16 arrays given as their raw 16-bit
patterns (numpy uint16).
"""
import ctypes
import os
import subprocess
import threading

import numpy as np

E4M3, E5M2 = 0, 1
RULE_CEIL, RULE_FLOOR = 0, 1
B_NK, B_KN = 0, 1
B_SCALE_BLOCK, B_SCALE_ROW = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()


def build():
    """Compile liboracle.so with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
                           _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.orc_decode.argtypes = [I, ctypes.c_uint8]
        lib.orc_decode.restype = ctypes.c_double
        lib.orc_encode.argtypes = [I, ctypes.c_double]
        lib.orc_encode.restype = ctypes.c_uint8
        lib.orc_scale_exp_ceil.argtypes = [I, ctypes.c_double]
        lib.orc_scale_exp_ceil.restype = I
        lib.orc_scale_exp_floor.argtypes = [I, ctypes.c_double]
        lib.orc_scale_exp_floor.restype = I
        for name in ("orc_quantize_rows", "orc_quantize_cols_t", "orc_quantize_block"):
            getattr(lib, name).argtypes = [P, I, I64, I64, I64, I, P, I64, P]
            getattr(lib, name).restype = None
        lib.orc_scale_f32.argtypes = [I, ctypes.c_float]
        lib.orc_scale_f32.restype = ctypes.c_float
        for name in ("orc_quantize_rows_f32s", "orc_quantize_cols_t_f32s", "orc_quantize_block_f32s"):
            getattr(lib, name).argtypes = [P, I, I64, I64, I64, I, P, I64, P]
            getattr(lib, name).restype = None
        lib.orc_gemm_f32s.argtypes = [I64, I64, I64, P, I64, I, P, P, I64, I, I, P, I, I64, I64, P, P, I64]
        lib.orc_gemm_f32s.restype = None
        lib.orc_gemm_f32s_elems.argtypes = [I64, I64, I64, P, I64, I, P, P, I64, I, I, P, I, P, P, I64, P, P]
        lib.orc_gemm_f32s_elems.restype = None
        lib.orc_mx_quantize.argtypes = [P, I, I64, I64, I64, I, I, P, I64, P, P]
        lib.orc_mx_quantize.restype = None
        lib.orc_gemm.argtypes = [I64, I64, I64, P, I64, I, P, P, I64, I, I, P, I,
                                 I64, I64, P, P, I64]
        lib.orc_gemm.restype = None
        lib.orc_gemm_elems.argtypes = [I64, I64, I64, P, I64, I, P, P, I64, I, I, P, I,
                                       P, P, I64, P, P]
        lib.orc_gemm_elems.restype = None
        lib.orc_mx_gemm.argtypes = [I64, I64, I64, P, I64, I, P, P, I64, I, P, I64, I64, P, P, I64]
        lib.orc_mx_gemm.restype = None
        lib.orc_mx_gemm_elems.argtypes = [I64, I64, I64, P, I64, I, P, P, I64, I, P, P, P, I64, P, P]
        lib.orc_mx_gemm_elems.restype = None
        U64 = ctypes.c_uint64
        lib.orc_philox4x64.argtypes = [P, P, P]
        lib.orc_philox4x64.restype = None
        lib.orc_gaussws_r.argtypes = [ctypes.c_uint32]
        lib.orc_gaussws_r.restype = I
        lib.orc_gaussws_noise.argtypes = [U64, U64, I64, I64, P]
        lib.orc_gaussws_noise.restype = None
        lib.orc_gaussws.argtypes = [P, I, I64, I64, I64, P, U64, U64, P, I64, I64, I64]
        lib.orc_gaussws.restype = None
        lib.orc_decode_array.argtypes = [I, P, I64, P]
        lib.orc_encode_array.argtypes = [I, P, I64, P]
        lib.orc_encode_f32_range.argtypes = [I, ctypes.c_uint32, I64, P]
        _lib = lib
        return lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(x):
    if x.dtype == np.float32:
        return 0, 4
    if x.dtype == np.uint16:
        return 1, 2
    raise TypeError("oracle inputs are float32 or bf16 bit patterns (uint16), got %s" % x.dtype)


def _split(n, threads):
    threads = max(1, min(int(threads), n)) if n > 0 else 1
    step = -(-n // threads) if n > 0 else 0
    return [(i, min(i + step, n)) for i in range(0, n, step)] if n > 0 else []


def _run(jobs):
    if len(jobs) <= 1:
        for j in jobs:
            j()
        return
    ts = [threading.Thread(target=j) for j in jobs]
    for t in ts:
        t.start()
    for t in ts:
        t.join()


def default_threads():
    return os.cpu_count() or 1


# ----------------------------------------------------------------------------- codec

def decode(fmt, codes):
    """fp64 values of FP8 codes (NaN where the format defines NaN)."""
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib.orc_decode_array(fmt, _ptr(c), c.size, _ptr(out))
    return out


def encode(fmt, x):
    """Saturating round-to-nearest-even FP8 codes of real values (fp64 input)."""
    lib = _load()
    v = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    lib.orc_encode_array(fmt, _ptr(v), v.size, _ptr(out))
    return out


def encode_f32_range(fmt, start, n):
    """Codes of the fp32 values with bit patterns start .. start+n-1."""
    lib = _load()
    out = np.empty(n, np.uint8)
    lib.orc_encode_f32_range(fmt, ctypes.c_uint32(start), n, _ptr(out))
    return out


def scale_exp_ceil(fmt, amax):
    return _load().orc_scale_exp_ceil(fmt, float(amax))


def scale_exp_floor(fmt, amax):
    return _load().orc_scale_exp_floor(fmt, float(amax))


# ------------------------------------------------------------------------ quantizers

def quantize_rows(x, fmt, threads=1):
    """1x128 groups along each row: returns (q [rows][cols] u8, s [rows][ceil(cols/128)] u8)."""
    lib = _load()
    x = np.ascontiguousarray(x)
    dt, es = _dtype_code(x)
    rows, cols = x.shape
    ng = -(-cols // 128)
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, ng), np.uint8)

    def job(r0, r1):
        return lambda: lib.orc_quantize_rows(
            ctypes.c_void_p(x.ctypes.data + r0 * cols * es), dt, r1 - r0, cols, cols, fmt,
            ctypes.c_void_p(q.ctypes.data + r0 * cols), cols, ctypes.c_void_p(s.ctypes.data + r0 * ng))
    _run([job(a, b) for a, b in _split(rows, threads)])
    return q, s


def quantize_cols_t(x, fmt, threads=1):
    """128-token groups down each column, transposed out:
    returns (qt [cols][rows] u8, st [cols][ceil(rows/128)] u8)."""
    lib = _load()
    x = np.ascontiguousarray(x)
    dt, es = _dtype_code(x)
    rows, cols = x.shape
    ng = -(-rows // 128)
    qt = np.empty((cols, rows), np.uint8)
    st = np.empty((cols, ng), np.uint8)

    def job(c0, c1):
        return lambda: lib.orc_quantize_cols_t(
            ctypes.c_void_p(x.ctypes.data + c0 * es), dt, rows, c1 - c0, cols, fmt,
            ctypes.c_void_p(qt.ctypes.data + c0 * rows), rows, ctypes.c_void_p(st.ctypes.data + c0 * ng))
    _run([job(a, b) for a, b in _split(cols, threads)])
    return qt, st


def quantize_block(w, fmt, threads=1):
    """128x128 tiles: returns (q [rows][cols] u8, s [ceil(rows/128)][ceil(cols/128)] u8)."""
    lib = _load()
    w = np.ascontiguousarray(w)
    dt, es = _dtype_code(w)
    rows, cols = w.shape
    nbr, nbc = -(-rows // 128), -(-cols // 128)
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((nbr, nbc), np.uint8)

    def job(i0, i1):
        r0, r1 = i0 * 128, min(i1 * 128, rows)
        return lambda: lib.orc_quantize_block(
            ctypes.c_void_p(w.ctypes.data + r0 * cols * es), dt, r1 - r0, cols, cols, fmt,
            ctypes.c_void_p(q.ctypes.data + r0 * cols), cols, ctypes.c_void_p(s.ctypes.data + i0 * nbc))
    _run([job(a, b) for a, b in _split(nbr, threads)])
    return q, s


def scale_f32(fmt, amax):
    """The fp32 scale amax / fmax of a group (1 when amax == 0)."""
    return np.float32(_load().orc_scale_f32(fmt, float(np.float32(amax))))


def quantize_rows_f32s(x, fmt, threads=1):
    """1x128 groups along rows with fp32 scales: (q u8, s float32 [rows][ceil(cols/128)])."""
    lib = _load()
    x = np.ascontiguousarray(x)
    dt, es = _dtype_code(x)
    rows, cols = x.shape
    ng = -(-cols // 128)
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, ng), np.float32)

    def job(r0, r1):
        return lambda: lib.orc_quantize_rows_f32s(
            ctypes.c_void_p(x.ctypes.data + r0 * cols * es), dt, r1 - r0, cols, cols, fmt,
            ctypes.c_void_p(q.ctypes.data + r0 * cols), cols, ctypes.c_void_p(s.ctypes.data + 4 * r0 * ng))
    _run([job(a, b) for a, b in _split(rows, threads)])
    return q, s


def quantize_cols_t_f32s(x, fmt, threads=1):
    """128-token groups down columns, transposed, fp32 scales: (qt u8 [cols][rows], st float32)."""
    lib = _load()
    x = np.ascontiguousarray(x)
    dt, es = _dtype_code(x)
    rows, cols = x.shape
    ng = -(-rows // 128)
    qt = np.empty((cols, rows), np.uint8)
    st = np.empty((cols, ng), np.float32)

    def job(c0, c1):
        return lambda: lib.orc_quantize_cols_t_f32s(
            ctypes.c_void_p(x.ctypes.data + c0 * es), dt, rows, c1 - c0, cols, fmt,
            ctypes.c_void_p(qt.ctypes.data + c0 * rows), rows, ctypes.c_void_p(st.ctypes.data + 4 * c0 * ng))
    _run([job(a, b) for a, b in _split(cols, threads)])
    return qt, st


def quantize_block_f32s(w, fmt, threads=1):
    """128x128 tiles with fp32 scales: (q u8, s float32 [ceil(rows/128)][ceil(cols/128)])."""
    lib = _load()
    w = np.ascontiguousarray(w)
    dt, es = _dtype_code(w)
    rows, cols = w.shape
    nbr, nbc = -(-rows // 128), -(-cols // 128)
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((nbr, nbc), np.float32)

    def job(i0, i1):
        r0, r1 = i0 * 128, min(i1 * 128, rows)
        return lambda: lib.orc_quantize_block_f32s(
            ctypes.c_void_p(w.ctypes.data + r0 * cols * es), dt, r1 - r0, cols, cols, fmt,
            ctypes.c_void_p(q.ctypes.data + r0 * cols), cols, ctypes.c_void_p(s.ctypes.data + 4 * i0 * nbc))
    _run([job(a, b) for a, b in _split(nbr, threads)])
    return q, s


def mx_quantize(x, fmt, rule=RULE_FLOOR, threads=1):
    """32-element blocks along rows: returns (q, s, counts) with s, counts [rows][ceil(cols/32)]."""
    lib = _load()
    x = np.ascontiguousarray(x)
    dt, es = _dtype_code(x)
    rows, cols = x.shape
    ng = -(-cols // 32)
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, ng), np.uint8)
    cnt = np.empty((rows, ng), np.uint8)

    def job(r0, r1):
        return lambda: lib.orc_mx_quantize(
            ctypes.c_void_p(x.ctypes.data + r0 * cols * es), dt, r1 - r0, cols, cols, fmt, rule,
            ctypes.c_void_p(q.ctypes.data + r0 * cols), cols, ctypes.c_void_p(s.ctypes.data + r0 * ng),
            ctypes.c_void_p(cnt.ctypes.data + r0 * ng))
    _run([job(a, b) for a, b in _split(rows, threads)])
    return q, s, cnt


# ------------------------------------------------------------------------------ GEMM

def _gemm_operands(a, sa, b, sb, b_layout):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    M, K = a.shape
    N = b.shape[0] if b_layout == B_NK else b.shape[1]
    if (b.shape[1] if b_layout == B_NK else b.shape[0]) != K:
        raise ValueError("A and B disagree on K")
    return a, sa, b, sb, M, N, K


def gemm(a, sa, a_fmt, b, sb, b_fmt, b_layout=B_NK, b_scale=B_SCALE_BLOCK, threads=1):
    """y = sum_k a(m,k) b(k,n) and t = sum_k |a(m,k) b(k,n)|, both fp64 [M][N]."""
    lib = _load()
    a, sa, b, sb, M, N, K = _gemm_operands(a, sa, b, sb, b_layout)
    y = np.empty((M, N), np.float64)
    t = np.empty((M, N), np.float64)
    ldb = b.shape[1]

    def job(m0, m1):
        return lambda: lib.orc_gemm(M, N, K, _ptr(a), K, a_fmt, _ptr(sa), _ptr(b), ldb, b_fmt, b_layout,
                                    _ptr(sb), b_scale, m0, m1, _ptr(y), _ptr(t), N)
    _run([job(m0, m1) for m0, m1 in _split(M, threads)])
    return y, t


def gemm_elems(a, sa, a_fmt, b, sb, b_fmt, ii, jj, b_layout=B_NK, b_scale=B_SCALE_BLOCK, threads=1):
    """The same sums for the listed output elements (ii[i], jj[i])."""
    lib = _load()
    a, sa, b, sb, M, N, K = _gemm_operands(a, sa, b, sb, b_layout)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    n = ii.size
    y = np.empty(n, np.float64)
    t = np.empty(n, np.float64)
    ldb = b.shape[1]

    def job(i0, i1):
        return lambda: lib.orc_gemm_elems(
            M, N, K, _ptr(a), K, a_fmt, _ptr(sa), _ptr(b), ldb, b_fmt, b_layout, _ptr(sb), b_scale,
            ctypes.c_void_p(ii.ctypes.data + 8 * i0), ctypes.c_void_p(jj.ctypes.data + 8 * i0), i1 - i0,
            ctypes.c_void_p(y.ctypes.data + 8 * i0), ctypes.c_void_p(t.ctypes.data + 8 * i0))
    _run([job(i0, i1) for i0, i1 in _split(n, threads)])
    return y, t


def _mx_operands(a, sa, b, sb):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("A and B disagree on K")
    nkc = -(-K // 32)
    if sa.shape != (M, nkc) or sb.shape != (N, nkc):
        raise ValueError("MX scales must be [rows][K/32]")
    return a, sa, b, sb, M, N, K


def mx_gemm(a, sa, a_fmt, b, sb, b_fmt, threads=1):
    """MX GEMM: A [M][K] with scales [M][K/32], B stored [N][K] with scales
    [N][K/32]; y = sum_k a(m,k) b(n,k), t = sum_k |a b|, fp64 [M][N]."""
    lib = _load()
    a, sa, b, sb, M, N, K = _mx_operands(a, sa, b, sb)
    y = np.empty((M, N), np.float64)
    t = np.empty((M, N), np.float64)

    def job(m0, m1):
        return lambda: lib.orc_mx_gemm(M, N, K, _ptr(a), K, a_fmt, _ptr(sa), _ptr(b), K, b_fmt, _ptr(sb),
                                       m0, m1, _ptr(y), _ptr(t), N)
    _run([job(m0, m1) for m0, m1 in _split(M, threads)])
    return y, t


def mx_gemm_elems(a, sa, a_fmt, b, sb, b_fmt, ii, jj, threads=1):
    """The MX sums for the listed output elements (ii[i], jj[i])."""
    lib = _load()
    a, sa, b, sb, M, N, K = _mx_operands(a, sa, b, sb)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    n = ii.size
    y = np.empty(n, np.float64)
    t = np.empty(n, np.float64)

    def job(i0, i1):
        return lambda: lib.orc_mx_gemm_elems(
            M, N, K, _ptr(a), K, a_fmt, _ptr(sa), _ptr(b), K, b_fmt, _ptr(sb),
            ctypes.c_void_p(ii.ctypes.data + 8 * i0), ctypes.c_void_p(jj.ctypes.data + 8 * i0), i1 - i0,
            ctypes.c_void_p(y.ctypes.data + 8 * i0), ctypes.c_void_p(t.ctypes.data + 8 * i0))
    _run([job(i0, i1) for i0, i1 in _split(n, threads)])
    return y, t


def _f32s_operands(a, sa, b, sb, b_layout):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    if np.asarray(sa).dtype != np.float32 or np.asarray(sb).dtype != np.float32:
        raise TypeError("fp32-scale GEMM: scales must be float32 arrays")
    sa = np.ascontiguousarray(sa)
    sb = np.ascontiguousarray(sb)
    M, K = a.shape
    N = b.shape[0] if b_layout == B_NK else b.shape[1]
    if (b.shape[1] if b_layout == B_NK else b.shape[0]) != K:
        raise ValueError("A and B disagree on K")
    return a, sa, b, sb, M, N, K


def gemm_f32s(a, sa, a_fmt, b, sb, b_fmt, b_layout=B_NK, b_scale=B_SCALE_BLOCK, threads=1):
    """GEMM over operands with fp32 scales (layouts of gemm, float32 instead of bytes):
    y = sum_k a(m,k) b(k,n), t = sum_k |a b|, fp64 [M][N]."""
    lib = _load()
    a, sa, b, sb, M, N, K = _f32s_operands(a, sa, b, sb, b_layout)
    y = np.empty((M, N), np.float64)
    t = np.empty((M, N), np.float64)
    ldb = b.shape[1]

    def job(m0, m1):
        return lambda: lib.orc_gemm_f32s(M, N, K, _ptr(a), K, a_fmt, _ptr(sa), _ptr(b), ldb, b_fmt, b_layout,
                                         _ptr(sb), b_scale, m0, m1, _ptr(y), _ptr(t), N)
    _run([job(m0, m1) for m0, m1 in _split(M, threads)])
    return y, t


def gemm_f32s_elems(a, sa, a_fmt, b, sb, b_fmt, ii, jj, b_layout=B_NK, b_scale=B_SCALE_BLOCK, threads=1):
    """gemm_f32s for the listed output elements (ii[i], jj[i])."""
    lib = _load()
    a, sa, b, sb, M, N, K = _f32s_operands(a, sa, b, sb, b_layout)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    n = ii.size
    y = np.empty(n, np.float64)
    t = np.empty(n, np.float64)
    ldb = b.shape[1]

    def job(i0, i1):
        return lambda: lib.orc_gemm_f32s_elems(
            M, N, K, _ptr(a), K, a_fmt, _ptr(sa), _ptr(b), ldb, b_fmt, b_layout, _ptr(sb), b_scale,
            ctypes.c_void_p(ii.ctypes.data + 8 * i0), ctypes.c_void_p(jj.ctypes.data + 8 * i0), i1 - i0,
            ctypes.c_void_p(y.ctypes.data + 8 * i0), ctypes.c_void_p(t.ctypes.data + 8 * i0))
    _run([job(i0, i1) for i0, i1 in _split(n, threads)])
    return y, t


# ------------------------------------------------------------------------- GaussWS

def philox4x64(ctr, key):
    """Philox4x64-10 of a 4-word counter and a 2-word key: four uint64."""
    lib = _load()
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.empty(4, np.uint64)
    lib.orc_philox4x64(_ptr(c), _ptr(k), _ptr(out))
    return out


def gaussws_r(u):
    """R in {-2..2} from 32 uniform bits."""
    return _load().orc_gaussws_r(int(u) & 0xFFFFFFFF)


def gaussws_noise(seed, stream, rows, cols):
    """R of every element of a [rows][cols] tensor (int8)."""
    lib = _load()
    out = np.empty((rows, cols), np.int8)
    lib.orc_gaussws_noise(seed, stream, rows, cols, _ptr(out))
    return out


def gaussws(w, bt, seed, stream, threads=1):
    """GaussWS sampled weight: bf16 bit patterns (uint16) [rows][cols] of
    w + R * max_bl|w| * 2^(1 - b_t); bt int8 [ceil(rows/32)][ceil(cols/32)]."""
    lib = _load()
    w = np.ascontiguousarray(w)
    dt, es = _dtype_code(w)
    rows, cols = w.shape
    bt = np.ascontiguousarray(bt, dtype=np.int8)
    nbr, nbc = -(-rows // 32), -(-cols // 32)
    if bt.shape != (nbr, nbc):
        raise ValueError("bitwidths must be [ceil(rows/32)][ceil(cols/32)]")
    out = np.empty((rows, cols), np.uint16)

    def job(i0, i1):
        return lambda: lib.orc_gaussws(_ptr(w), dt, rows, cols, cols, _ptr(bt), seed, stream, _ptr(out), cols,
                                       i0, i1)
    _run([job(a, b) for a, b in _split(nbr, threads)])
    return out
