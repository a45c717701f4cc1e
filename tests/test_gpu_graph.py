"""The entry points inside a captured HIP graph (how the benchmark times a
step): each replay, with other eager work and synchronisations between the
replays, must reproduce the eager step's outputs bit for bit.  The library
allocates, frees and synchronises nothing and issues no memsets, so its
launches are safe to capture."""
import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import synth
from gpu_helpers import dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    x = dev(synth.activations_like(1, (512, 1024), bf16=True))
    w = dev(synth.weights_like(2, (768, 1024), bf16=True))
    wf = dev(synth.weights_like(3, (256, 512), bf16=False))
    u8 = dict(dtype=torch.uint8, device="cuda")
    xq, xs = torch.empty((512, 1024), **u8), torch.empty((512, 8), **u8)
    xqt, xst = torch.empty((1024, 512), **u8), torch.empty((1024, 4), **u8)
    wq, ws = torch.empty((768, 1024), **u8), torch.empty((6, 8), **u8)
    mq, ms = torch.empty((512, 1024), **u8), torch.empty((512, 32), **u8)
    nq, ns = torch.empty((768, 1024), **u8), torch.empty((768, 32), **u8)
    y = torch.empty((512, 768), dtype=torch.bfloat16, device="cuda")
    ym = torch.empty((512, 768), dtype=torch.float32, device="cuda")
    bt = torch.full((8, 16), 6, dtype=torch.int8, device="cuda")
    wh = torch.empty((256, 512), dtype=torch.bfloat16, device="cuda")
    outs = [xq, xs, xqt, xst, wq, ws, mq, ms, nq, ns, y, ym, wh]

    def step():
        s = torch.cuda.current_stream().cuda_stream
        assert mx.fp8_quantize_token_dual(x.data_ptr(), mx.BF16, 512, 1024, 1024, mx.E4M3, xq.data_ptr(), 1024,
                                          xs.data_ptr(), xqt.data_ptr(), 512, xst.data_ptr(), s) == 0
        assert mx.fp8_quantize_block(w.data_ptr(), mx.BF16, 768, 1024, 1024, mx.E4M3, wq.data_ptr(), 1024,
                                     ws.data_ptr(), s) == 0
        assert mx.fp8_block_scaled_gemm(512, 768, 1024, xq.data_ptr(), 1024, mx.E4M3, xs.data_ptr(), wq.data_ptr(),
                                        1024, mx.E4M3, mx.B_NK, ws.data_ptr(), mx.SCALE_BLOCK128, y.data_ptr(), 768,
                                        mx.BF16, s) == 0
        assert mx.mx_quantize(x.data_ptr(), mx.BF16, 512, 1024, 1024, mx.E4M3, mx.RULE_FLOOR, mq.data_ptr(), 1024,
                              ms.data_ptr(), None, s) == 0
        assert mx.mx_quantize(w.data_ptr(), mx.BF16, 768, 1024, 1024, mx.E4M3, mx.RULE_FLOOR, nq.data_ptr(), 1024,
                              ns.data_ptr(), None, s) == 0
        assert mx.mx_gemm(512, 768, 1024, mq.data_ptr(), 1024, mx.E4M3, ms.data_ptr(), nq.data_ptr(), 1024, mx.E4M3,
                          ns.data_ptr(), ym.data_ptr(), 768, mx.F32, s) == 0
        assert mx.gaussws_sample(wf.data_ptr(), mx.F32, 256, 512, 512, bt.data_ptr(), 9, 1, wh.data_ptr(), 512,
                                 s) == 0

    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for replay in range(4):
        for o in outs:
            o.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # other eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), "replay %d, output %d differs from the eager step" % (replay, i)
