"""The tensor conveniences of the Python binding reject mismatched tensors before
any pointer reaches the C ABI (which cannot see extents): wrong dtype, wrong
shape, non-unit column stride, non-contiguous scales, K extents that disagree,
and tensors off the current CUDA device.  CPU tensors reach every shape and
dtype check first and then fail the device check, so all of this runs without
a GPU."""
import pytest
import torch

import mx_block_scaled_x128_amd as mx

u8, f32, bf16 = torch.uint8, torch.float32, torch.bfloat16


def codes(r, c):
    return torch.zeros((r, c), dtype=u8)


def good_gemm(b_layout=mx.B_NK, b_scale=mx.SCALE_BLOCK128, M=64, N=200, K=256):
    a, sa = codes(M, K), codes(M, K // 128)
    if b_layout == mx.B_NK:
        b = codes(N, K)
        sb = codes(N, K // 128) if b_scale == mx.SCALE_ROW128 else codes((N + 127) // 128, K // 128)
    else:
        b, sb = codes(K, N), codes(K // 128, (N + 127) // 128)
    return a, sa, b, sb


def raises(match, fn, *args, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


@pytest.mark.parametrize("b_layout,b_scale", [(mx.B_NK, mx.SCALE_BLOCK128), (mx.B_KN, mx.SCALE_BLOCK128),
                                              (mx.B_NK, mx.SCALE_ROW128)])
def test_gemm_well_formed_cpu_operands_fail_only_on_device(b_layout, b_scale):
    a, sa, b, sb = good_gemm(b_layout, b_scale)
    raises("CUDA tensor", mx.block_scaled_gemm, a, sa, 0, b, sb, 0, b_layout, b_scale)
    raises("CUDA tensor", mx.gemm_f32s, a, sa.float(), 0, b, sb.float(), 0, b_layout, b_scale)


def test_gemm_rejects_k_mismatch_and_bad_shapes():
    a, sa, b, sb = good_gemm()
    raises("b must have shape", mx.block_scaled_gemm, a, sa, 0, codes(200, 384), sb, 0)
    a2, sa2, b2, sb2 = good_gemm(mx.B_KN)
    raises("b must have shape", mx.block_scaled_gemm, a2, sa2, 0, codes(384, 200), sb2, 0, mx.B_KN)
    # a strided view whose K extent is below a's
    wide = codes(200, 512)
    raises("b must have shape", mx.block_scaled_gemm, a, sa, 0, wide[:, :128], sb, 0)
    raises("K must be a multiple of 128", mx.block_scaled_gemm, codes(64, 200), sa, 0, codes(200, 200), sb, 0)
    raises("a_scales must have shape", mx.block_scaled_gemm, a, codes(64, 3), 0, b, sb, 0)
    raises("b_scales must have shape", mx.block_scaled_gemm, a, sa, 0, b, codes(200, 2), 0)
    raises("b_scales must have shape", mx.block_scaled_gemm, a, sa, 0, b, codes(2, 2), 0, mx.B_NK,
           mx.SCALE_ROW128)
    raises("b_scales must have shape", mx.block_scaled_gemm, a2, sa2, 0, b2, codes(2, 2).t().contiguous()[:, :1],
           0, mx.B_KN)


def test_gemm_rejects_dtypes_strides_and_layout_combinations():
    a, sa, b, sb = good_gemm()
    raises("a must have dtype", mx.block_scaled_gemm, a.float(), sa, 0, b, sb, 0)
    raises("a_scales must have dtype", mx.block_scaled_gemm, a, sa.float(), 0, b, sb, 0)
    # uint8 scales given to the fp32-scale GEMM would be read as 4x the bytes
    raises("a_scales must have dtype", mx.gemm_f32s, a, sa, 0, b, sb.float(), 0)
    raises("b_scales must have dtype", mx.gemm_f32s, a, sa.float(), 0, b, sb, 0)
    # transposed (non-contiguous) scales
    sq = codes(2, 2)
    raises("b_scales must (be contiguous|have unit column stride)", mx.block_scaled_gemm, codes(64, 256), codes(64, 2), 0, codes(256, 256),
           sq.t(), 0)
    raises("a must have unit column stride", mx.block_scaled_gemm, codes(256, 64).t(), sa, 0, b, sb, 0)
    raises("per-row B scales need B stored", mx.block_scaled_gemm, a, sa, 0, b, sb, 0, mx.B_KN, mx.SCALE_ROW128)
    raises("b_layout", mx.block_scaled_gemm, a, sa, 0, b, sb, 0, 7)
    raises("b_scale_mode", mx.block_scaled_gemm, a, sa, 0, b, sb, 0, mx.B_NK, 9)
    raises("out must have shape", mx.block_scaled_gemm, a, sa, 0, b, sb, 0, out=torch.zeros(64, 199))
    raises("out must have dtype", mx.block_scaled_gemm, a, sa, 0, b, sb, 0, out=torch.zeros(64, 200,
                                                                                          dtype=torch.float16))
    raises("out_dtype", mx.block_scaled_gemm, a, sa, 0, b, sb, 0, out_dtype=torch.float16)


def test_float8_views_are_accepted_as_codes():
    a, sa, b, sb = good_gemm()
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8 dtypes")
    raises("CUDA tensor", mx.block_scaled_gemm, a.view(torch.float8_e4m3fn), sa, 0, b.view(torch.float8_e5m2),
           sb, 1)


def test_mx_gemm_rejects_bad_scales():
    a, b = codes(64, 256), codes(96, 256)
    raises("CUDA tensor", mx.mx_scaled_gemm, a, codes(64, 8), 0, b, codes(96, 8), 0)
    raises("a_scales must have shape", mx.mx_scaled_gemm, a, codes(64, 2), 0, b, codes(96, 8), 0)
    raises("b_scales must have shape", mx.mx_scaled_gemm, a, codes(64, 8), 0, b, codes(64, 8), 0)
    raises("b must have shape", mx.mx_scaled_gemm, a, codes(64, 8), 0, codes(96, 384), codes(96, 8), 0)
    raises("b_scales must have dtype", mx.mx_scaled_gemm, a, codes(64, 8), 0, b, codes(96, 8).float(), 0)


def test_quantizers_reject_inputs():
    raises("x must be a 2-D", mx.quantize_token, torch.zeros(4, 4, 4))
    raises("x must have dtype", mx.quantize_token, torch.zeros(4, 128, dtype=torch.float16))
    raises("x must have unit column stride", mx.quantize_token, torch.zeros(128, 64).t())
    raises("CUDA tensor", mx.quantize_token, torch.zeros(4, 128))
    raises("CUDA tensor", mx.quantize_block, torch.zeros(4, 128, dtype=bf16))
    raises("CUDA tensor", mx.quantize_token_dual, torch.zeros(16, 128))
    raises("CUDA tensor", mx.quantize_block_dual, torch.zeros(16, 128))
    raises("CUDA tensor", mx.quantize_token_f32s, torch.zeros(4, 128))
    raises("CUDA tensor", mx.quantize_block_f32s, torch.zeros(4, 128))
    raises("multiple of 32", mx.quantize_mx, torch.zeros(4, 48))
    raises("CUDA tensor", mx.quantize_mx, torch.zeros(4, 64))


def test_gaussws_rejects_bitwidths_and_out():
    w = torch.zeros(40, 64)
    raises("bitwidths must have shape", mx.gaussws, w, torch.zeros((1, 2), dtype=torch.int8), 1)
    raises("bitwidths must have dtype", mx.gaussws, w, torch.zeros((2, 2), dtype=torch.uint8), 1)
    raises("out must have dtype", mx.gaussws, w, torch.zeros((2, 2), dtype=torch.int8), 1, out=torch.zeros(40, 64))
    raises("CUDA tensor", mx.gaussws, w, torch.zeros((2, 2), dtype=torch.int8), 1)
