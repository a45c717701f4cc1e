"""Every entry point runs on the stream it is given: the current torch stream when
the wrapper's `stream` is None, else the given one.  Inputs are produced on a side
stream behind a queue of slow elementwise work, so a kernel launched on another
stream would read them before they exist; the results must equal those computed
on the default stream, bit for bit.  Calls go through the C ABI."""
import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import synth
from gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _busy(stream, n=40):
    """Queues a few milliseconds of elementwise work on `stream`."""
    with torch.cuda.stream(stream):
        t = torch.ones(16 << 20, dtype=torch.float32, device="cuda")
        for _ in range(n):
            t.mul_(1.0001)
    return t


def _reference(x, w):
    q, s = mx.quantize_token(x, mx.E4M3, mx.ROW)
    qt, st = mx.quantize_token(x, mx.E4M3, mx.COL_T)
    qw, sw = mx.quantize_block(w, mx.E4M3)
    y = mx.block_scaled_gemm(q, s, mx.E4M3, qw, sw, mx.E4M3, out_dtype=torch.float32)
    qm, sm, cm = mx.quantize_mx(x.float(), mx.E4M3, mx.RULE_FLOOR)
    g = mx.gaussws(w, torch.full((w.shape[0] // 32, w.shape[1] // 32), 6, dtype=torch.int8, device="cuda"), 11, 2)
    torch.cuda.synchronize()
    return [q, s, qt, st, qw, sw, y, qm, sm, cm, g]


def _inputs():
    x = dev(synth.activations_like(6100, (1024, 2048), bf16=True))
    w = dev(synth.weights_like(6101, (1024, 2048), bf16=True))
    return x, w


def _same(a, b):
    for u, v in zip(a, b):
        assert u.dtype == v.dtype and u.shape == v.shape
        assert torch.equal(u.view(torch.uint8) if u.dtype == torch.float32 else u,
                           v.view(torch.uint8) if v.dtype == torch.float32 else v)


def test_current_side_stream():
    x, w = _inputs()
    ref = _reference(x, w)
    s = torch.cuda.Stream()
    keep = _busy(s)
    with torch.cuda.stream(s):
        x2, w2 = x.clone(), w.clone()   # ready only after the queued work
        q, sc = mx.quantize_token(x2, mx.E4M3, mx.ROW)
        qt, st = mx.quantize_token(x2, mx.E4M3, mx.COL_T)
        qw, sw = mx.quantize_block(w2, mx.E4M3)
        y = mx.block_scaled_gemm(q, sc, mx.E4M3, qw, sw, mx.E4M3, out_dtype=torch.float32)
        qm, sm, cm = mx.quantize_mx(x2.float(), mx.E4M3, mx.RULE_FLOOR)
        g = mx.gaussws(w2, torch.full((32, 64), 6, dtype=torch.int8, device="cuda"), 11, 2)
    s.synchronize()
    del keep
    _same(ref, [q, sc, qt, st, qw, sw, y, qm, sm, cm, g])


def test_explicit_stream_argument():
    x, w = _inputs()
    ref = _reference(x, w)
    s = torch.cuda.Stream()
    keep = _busy(s)
    with torch.cuda.stream(s):
        x2, w2 = x.clone(), w.clone()
        x2f = x2.float()
        bt = torch.full((32, 64), 6, dtype=torch.int8, device="cuda")
    # The current stream is the default one again; every call names s.
    q, sc = mx.quantize_token(x2, mx.E4M3, mx.ROW, stream=s)
    qt, st = mx.quantize_token(x2, mx.E4M3, mx.COL_T, stream=s)
    qw, sw = mx.quantize_block(w2, mx.E4M3, stream=s)
    y = mx.block_scaled_gemm(q, sc, mx.E4M3, qw, sw, mx.E4M3, out_dtype=torch.float32, stream=s)
    qm, sm, cm = mx.quantize_mx(x2f, mx.E4M3, mx.RULE_FLOOR, stream=s)
    g = mx.gaussws(w2, bt, 11, 2, stream=s)
    s.synchronize()
    del keep
    _same(ref, [q, sc, qt, st, qw, sw, y, qm, sm, cm, g])
