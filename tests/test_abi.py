"""C-ABI tests that need no GPU: the library loads, exports every function that
include/mxfp8.h declares, and rejects every invalid argument with the documented
status before any HIP call (fake, never-dereferenced pointers)."""
import os
import re

import pytest

import mx_block_scaled_x128_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp8.h")

OK, NULL, SHAPE, LD, ALIGN, ENUM, ALIAS = 0, 1, 2, 3, 4, 5, 6
X, Q, S, C, P2 = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000  # fake aligned device pointers
MIS = 0x200008  # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = mx.load_library()
    names = declared_functions()
    assert set(names) >= {"fp8_quantize_token", "fp8_quantize_block", "mx_quantize", "fp8_block_scaled_gemm",
                          "mx_gemm", "fp8_quantize_token_dual", "fp8_quantize_block_dual",
                          "fp8_quantize_token_f32s", "fp8_quantize_block_f32s", "fp8_gemm_f32s",
                          "gaussws_sample",
                          "mxfp8_status_string", "mxfp8_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert mx.mxfp8_version() == 100
    for st in range(8):
        assert mx.mxfp8_status_string(st)
    assert mx.mxfp8_status_string(99) == "unknown status"


def tok(x=X, dt=1, rows=256, cols=512, ldx=512, axis=0, fmt=0, q=Q, ldq=512, s=S):
    return mx.fp8_quantize_token(x, dt, rows, cols, ldx, axis, fmt, q, ldq, s, None)


def test_token_validation():
    assert tok(dt=2) == ENUM
    assert tok(axis=2) == ENUM
    assert tok(fmt=7) == ENUM
    assert tok(rows=-1) == SHAPE
    assert tok(rows=0) == OK and tok(cols=0, x=None, q=None, s=None) == OK  # empty: no launch
    assert tok(x=None) == NULL and tok(q=None) == NULL and tok(s=None) == NULL
    assert tok(ldx=500) == LD and tok(ldx=520) == LD and tok(ldq=500) == LD
    assert tok(cols=520, ldx=528, ldq=528) == SHAPE  # cols % 16
    assert tok(x=MIS) == ALIGN and tok(q=MIS) == ALIGN
    assert tok(q=X) == ALIAS and tok(s=X) == ALIAS and tok(s=Q) == ALIAS
    # COL_T: q is [cols][rows]; rows must be a multiple of 16
    assert tok(axis=1, rows=256, cols=512, ldx=512, ldq=240) == LD
    assert tok(axis=1, rows=136, cols=512, ldx=512, ldq=144) == SHAPE
    assert tok(rows=2 ** 31, ldx=512) == SHAPE


def blk(w=X, dt=0, rows=256, cols=512, ldw=512, fmt=1, q=Q, ldq=512, s=S):
    return mx.fp8_quantize_block(w, dt, rows, cols, ldw, fmt, q, ldq, s, None)


def test_block_validation():
    assert blk(dt=-1) == ENUM and blk(fmt=2) == ENUM
    assert blk(cols=-16) == SHAPE and blk(cols=24, ldw=32, ldq=32) == SHAPE
    assert blk(rows=0, w=None) == OK
    assert blk(w=None) == NULL
    assert blk(ldw=16) == LD and blk(ldq=520) == LD
    assert blk(w=MIS) == ALIGN
    assert blk(q=X) == ALIAS


def test_f32s_validation():
    def tok(x=X, dt=1, rows=256, cols=512, ldx=512, axis=0, fmt=0, q=Q, ldq=512, s=S):
        return mx.fp8_quantize_token_f32s(x, dt, rows, cols, ldx, axis, fmt, q, ldq, s, None)

    def blk(w=X, dt=0, rows=256, cols=512, ldw=512, fmt=1, q=Q, ldq=512, s=S):
        return mx.fp8_quantize_block_f32s(w, dt, rows, cols, ldw, fmt, q, ldq, s, None)

    def g(M=256, N=256, K=512, a=X, lda=512, afmt=0, sa=S, b=Q, ldb=512, bfmt=0, blay=0, sb=P2, bsm=0, c=C,
          ldc=256, cdt=0):
        return mx.fp8_gemm_f32s(M, N, K, a, lda, afmt, sa, b, ldb, bfmt, blay, sb, bsm, c, ldc, cdt, None)
    assert tok(axis=3) == ENUM and tok(fmt=2) == ENUM and tok(dt=2) == ENUM
    assert tok(rows=-1) == SHAPE and tok(cols=520, ldx=528, ldq=528) == SHAPE
    assert tok(axis=1, rows=136, cols=512, ldx=512, ldq=144) == SHAPE
    assert tok(s=None) == NULL and tok(ldq=500) == LD and tok(x=MIS) == ALIGN and tok(s=S + 2) == ALIGN
    assert tok(q=X) == ALIAS and tok(rows=0) == OK
    assert blk(fmt=5) == ENUM and blk(cols=24, ldw=32, ldq=32) == SHAPE and blk(w=None) == NULL
    assert blk(s=S + 1) == ALIGN and blk(s=X) == ALIAS and blk(cols=0) == OK
    assert g(afmt=2) == ENUM and g(blay=2) == ENUM and g(bsm=2) == ENUM and g(cdt=2) == ENUM
    assert g(blay=1, bsm=1, ldb=256) == ENUM
    assert g(K=200) == SHAPE and g(M=-1) == SHAPE and g(M=0) == OK and g(N=0, c=None) == OK
    assert g(c=None) == NULL and g(sa=None) == NULL and g(sb=None) == NULL
    assert g(lda=256) == LD and g(ldb=500) == LD and g(ldc=200) == LD and g(blay=1, ldb=128) == LD
    assert g(lda=(1 << 24) + 16) == LD
    assert g(a=MIS) == ALIGN and g(c=MIS) == ALIGN and g(sa=S + 2) == ALIGN and g(sb=P2 + 3) == ALIGN
    assert g(c=X) == ALIAS and g(c=S) == ALIAS and g(c=P2) == ALIAS


def test_gaussws_validation():
    def call(w=X, dt=0, rows=64, cols=256, ldw=256, bt=S, out=Q, ldo=256):
        return mx.gaussws_sample(w, dt, rows, cols, ldw, bt, 1, 2, out, ldo, None)
    assert call(dt=2) == ENUM
    assert call(rows=-1) == SHAPE and call(cols=250, ldw=256, ldo=256) == SHAPE and call(rows=2 ** 31) == SHAPE
    assert call(rows=0, w=None, bt=None, out=None) == OK and call(cols=0) == OK
    assert call(w=None) == NULL and call(bt=None) == NULL and call(out=None) == NULL
    assert call(ldw=240) == LD and call(ldw=264) == LD and call(ldo=250) == LD
    assert call(w=MIS) == ALIGN and call(out=MIS) == ALIGN
    assert call(out=X) == ALIAS and call(out=S) == ALIAS


Q2, S2 = 0x600000, 0x700000


@pytest.mark.parametrize("fn", ["fp8_quantize_token_dual", "fp8_quantize_block_dual"])
def test_dual_validation(fn):
    f = getattr(mx, fn)

    def call(x=X, dt=1, rows=256, cols=512, ldx=512, fmt=0, q=Q, ldq=512, s=S, qt=Q2, ldqt=256, st=S2):
        return f(x, dt, rows, cols, ldx, fmt, q, ldq, s, qt, ldqt, st, None)
    assert call(fmt=2) == ENUM and call(dt=3) == ENUM
    assert call(rows=-16) == SHAPE and call(rows=2 ** 31) == SHAPE
    assert call(rows=0, x=None, q=None, qt=None) == OK and call(cols=0, s=None, st=None) == OK
    assert call(rows=136, ldqt=144) == SHAPE and call(cols=520, ldx=528, ldq=528) == SHAPE
    assert call(x=None) == NULL and call(q=None) == NULL and call(qt=None) == NULL and call(st=None) == NULL
    assert call(ldx=500) == LD and call(ldq=500) == LD and call(ldqt=240) == LD and call(ldqt=264) == LD
    assert call(x=MIS) == ALIGN and call(qt=MIS) == ALIGN
    assert call(q=X) == ALIAS and call(qt=X) == ALIAS and call(st=X) == ALIAS
    assert call(qt=Q) == ALIAS and call(st=Q) == ALIAS and call(qt=S) == ALIAS and call(st=S) == ALIAS


def mxq(x=X, dt=0, rows=64, cols=256, ldx=256, fmt=0, rule=1, q=Q, ldq=256, s=S, cnt=P2):
    return mx.mx_quantize(x, dt, rows, cols, ldx, fmt, rule, q, ldq, s, cnt, None)


def test_mx_validation():
    assert mxq(rule=2) == ENUM and mxq(fmt=3) == ENUM and mxq(dt=5) == ENUM
    assert mxq(cols=48, ldx=48, ldq=48) == SHAPE
    assert mxq(s=None) == NULL
    assert mxq(ldq=255) == LD
    assert mxq(cnt=X) == ALIAS and mxq(cnt=Q) == ALIAS and mxq(cnt=S) == ALIAS
    assert mxq(x=MIS) == ALIGN
    assert mxq(rows=0) == OK


def gemm(M=256, N=256, K=512, a=X, lda=512, afmt=0, sa=S, b=Q, ldb=512, bfmt=0, blay=0, sb=P2, bsm=0, c=C,
         ldc=256, cdt=0):
    return mx.fp8_block_scaled_gemm(M, N, K, a, lda, afmt, sa, b, ldb, bfmt, blay, sb, bsm, c, ldc, cdt, None)


def test_gemm_validation():
    assert gemm(afmt=2) == ENUM and gemm(bfmt=-1) == ENUM and gemm(blay=2) == ENUM
    assert gemm(bsm=2) == ENUM and gemm(cdt=3) == ENUM
    assert gemm(blay=1, bsm=1, ldb=256) == ENUM  # per-row B scales only with [N][K] storage
    assert gemm(K=500) == SHAPE and gemm(M=-1) == SHAPE
    assert gemm(M=0) == OK and gemm(N=0, c=None) == OK
    assert gemm(c=None) == NULL and gemm(a=None) == NULL and gemm(sb=None) == NULL
    assert gemm(lda=256) == LD and gemm(ldb=500) == LD and gemm(ldc=200) == LD
    assert gemm(blay=1, ldb=128) == LD  # KN: ldb >= N
    assert gemm(lda=(1 << 24) + 16) == LD and gemm(ldb=(1 << 24) + 16) == LD  # 32-bit tile offsets
    assert gemm(a=MIS) == ALIGN and gemm(c=MIS) == ALIGN
    assert gemm(c=X) == ALIAS and gemm(c=S) == ALIAS


def mxg(M=256, N=256, K=512, a=X, lda=512, afmt=0, sa=S, b=Q, ldb=512, bfmt=0, sb=P2, c=C, ldc=256, cdt=0):
    return mx.mx_gemm(M, N, K, a, lda, afmt, sa, b, ldb, bfmt, sb, c, ldc, cdt, None)


def test_mx_gemm_validation():
    assert mxg(afmt=2) == ENUM and mxg(bfmt=-1) == ENUM and mxg(cdt=2) == ENUM
    assert mxg(K=480) == SHAPE and mxg(K=32) == SHAPE and mxg(N=-1) == SHAPE and mxg(M=2 ** 31) == SHAPE
    assert mxg(M=0, a=None, sa=None) == OK and mxg(N=0, c=None) == OK
    assert mxg(c=None) == NULL and mxg(b=None) == NULL and mxg(sa=None) == NULL and mxg(sb=None) == NULL
    assert mxg(lda=496) == LD and mxg(ldb=520) == LD and mxg(ldc=255) == LD
    assert mxg(lda=(1 << 24) + 16) == LD and mxg(ldb=(1 << 24) + 16) == LD
    assert mxg(a=MIS) == ALIGN and mxg(c=MIS) == ALIGN
    assert mxg(sa=S + 2) == ALIGN and mxg(sb=P2 + 1) == ALIGN
    assert mxg(c=X) == ALIAS and mxg(c=Q) == ALIAS and mxg(c=S) == ALIAS and mxg(c=P2) == ALIAS


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mx, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(mx, "_lib", None)
    with pytest.raises(ImportError):
        mx.load_library()
