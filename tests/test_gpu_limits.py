"""Maximum sizes.  Quantizer inputs past 4 GiB (an 8 GiB bf16 input of 2^27 rows, so
that byte offsets and row counts exceed 32 bits where the kernels form 64-bit
addresses), and the GEMM at the largest leading dimension the C ABI accepts, 2^24
bytes, on the 256x256 tile path, where a tile's 32-bit lane offsets reach
255 * 2^24 (A stored [M][K]) or 127 * 2^24 + N (B stored [K][N]).

The large quantizer input repeats one seeded 4096-row block, so each 4096-row
slice of the output must equal the oracle's output for that block; slices at the
start, the middle and the end are compared.  The GEMM operands are N(0, 1) data
quantized on the GPU and copied into buffers with the maximal row pitch; every
output is compared with the oracle at the plain bound.  Calls go through the C ABI."""
import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import oracle
import synth
from gpu_helpers import ORACLE_THREADS, assert_gemm_close, dev, host

pytestmark = pytest.mark.gpu

BLOCK, REPEAT, COLS = 4096, 1 << 15, 32     # 2^27 rows x 32 bf16 = 8 GiB
LD_MAX = 1 << 24


@pytest.fixture(scope="module")
def big():
    small = synth.heavy_tail_like(6200, (BLOCK, COLS), bf16=True)
    x = dev(small).repeat(REPEAT, 1)
    assert x.shape == (BLOCK * REPEAT, COLS) and x.numel() * 2 == 8 << 30
    yield small, x
    del x
    torch.cuda.empty_cache()


def _slices(n_blocks):
    return [0, n_blocks // 2, n_blocks - 1]


def test_token_rows_past_4gib(big):
    small, x = big
    q, s = mx.quantize_token(x, mx.E5M2, mx.ROW)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows(small, oracle.E5M2)
    qv, sv = q.view(REPEAT, BLOCK, COLS), s.view(REPEAT, BLOCK, 1)
    for k in _slices(REPEAT):
        assert np.array_equal(host(qv[k]), q_ref)
        assert np.array_equal(host(sv[k]), s_ref)


def test_token_cols_t_past_4gib(big):
    small, x = big
    qt, st = mx.quantize_token(x, mx.E4M3, mx.COL_T)
    torch.cuda.synchronize()
    qt_ref, st_ref = oracle.quantize_cols_t(small, oracle.E4M3)
    for k in _slices(REPEAT):
        assert np.array_equal(host(qt[:, k * BLOCK:(k + 1) * BLOCK]), qt_ref)
        assert np.array_equal(host(st[:, k * (BLOCK // 128):(k + 1) * (BLOCK // 128)]), st_ref)


def test_block_past_4gib(big):
    small, x = big
    q, s = mx.quantize_block(x, mx.E4M3)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_block(small, oracle.E4M3)
    for k in _slices(REPEAT):
        assert np.array_equal(host(q[k * BLOCK:(k + 1) * BLOCK]), q_ref)
        assert np.array_equal(host(s[k * (BLOCK // 128):(k + 1) * (BLOCK // 128)]), s_ref)


def _pitched(codes, ld):
    """The codes in a buffer whose rows are ld bytes apart (a strided view)."""
    buf = torch.empty((codes.shape[0], ld), dtype=torch.uint8, device="cuda")
    v = buf[:, :codes.shape[1]]
    v.copy_(codes)
    return v


@pytest.mark.parametrize("bf16_out", [False, True])
def test_gemm_a_at_max_leading_dimension(bf16_out):
    """M = 256 (one 256-row tile row), N = 33024 (more 128x128 tiles than two per CU,
    so 256x256 tiles), K = 256, A's rows 2^24 bytes apart."""
    M, N, K = 256, 33024, 256
    rng = np.random.default_rng(6201)
    aq, a_s = mx.quantize_token(dev(rng.standard_normal((M, K)).astype(np.float32)), mx.E4M3, mx.ROW)
    bq, b_s = mx.quantize_block(dev(rng.standard_normal((N, K)).astype(np.float32)), mx.E4M3)
    a_far = _pitched(aq, LD_MAX)
    assert a_far.stride(0) == LD_MAX
    y = mx.block_scaled_gemm(a_far, a_s, mx.E4M3, bq, b_s, mx.E4M3,
                             out_dtype=torch.bfloat16 if bf16_out else torch.float32)
    torch.cuda.synchronize()
    del a_far
    torch.cuda.empty_cache()
    y_ref, t_ref = oracle.gemm(host(aq), host(a_s), 0, host(bq), host(b_s), 0, threads=ORACLE_THREADS)
    assert_gemm_close(host(y), y_ref, t_ref, bf16_out, "lda = 2^24")


def test_gemm_b_kn_at_max_leading_dimension():
    """B stored [K][N] with rows 2^24 bytes apart, on 256x256 tiles (M = 256,
    N = 33024, K = 256)."""
    M, N, K = 256, 33024, 256
    rng = np.random.default_rng(6202)
    aq, a_s = mx.quantize_token(dev(rng.standard_normal((M, K)).astype(np.float32)), mx.E4M3, mx.ROW)
    # B [K][N] with 128x128 block scales [K/128][N/128]: the block quantization of B itself.
    bq, b_s = mx.quantize_block(dev(rng.standard_normal((K, N)).astype(np.float32)), mx.E4M3)
    b_far = _pitched(bq, LD_MAX)
    y = mx.block_scaled_gemm(aq, a_s, mx.E4M3, b_far, b_s, mx.E4M3, mx.B_KN, mx.SCALE_BLOCK128,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    del b_far
    torch.cuda.empty_cache()
    y_ref, t_ref = oracle.gemm(host(aq), host(a_s), 0, host(bq), host(b_s), 0, oracle.B_KN, oracle.B_SCALE_BLOCK,
                               threads=ORACLE_THREADS)
    assert_gemm_close(host(y), y_ref, t_ref, False, "ldb = 2^24, B [K][N]")
