"""bf16 output is the fp32 result rounded to nearest-even.  For the same operands
a GEMM's bf16 output must equal the CPU's round-to-nearest-even of its fp32
output bit for bit: both come from one accumulation, only the epilogue differs.

Rows of A come in four bands (row index mod 4), against B block scales that
alternate small and large by column block, so the results land among normal
values, among fp32 subnormals (bf16 has fp32's exponent range, so they stay
subnormal), next to the top of the range (where rounding carries into
infinity, and fp32 itself overflows), and, from rows with two nonzero codes,
on exact halfway cases of the bf16 rounding.  B's codes and the top band's
codes are positive, so no sum meets infinities of both signs.

The block-scaled GEMM on 128x128 tiles, on one round of 256x256 tiles and on a
round with a quadrant tail, both B layouts; the MX and the fp32-scale GEMMs,
which share the epilogue.  Calls go through the C ABI."""
import numpy as np
import pytest
import torch

import mx_block_scaled_x128_amd as mx
import synth
from gpu_helpers import dev

pytestmark = pytest.mark.gpu

# 128x128 tiles; one round of 256x256 tiles on 256 compute units; 17 x 16 tiles,
# whose short last round runs as quadrants.
SHAPES = [(640, 384, 512), (4096, 4096, 512), (4352, 4096, 512)]

A_BANDS = [(120, 134), (10, 16), (200, 215), (127, 127)]   # E8M0 bytes per band
B_SMALL, B_LARGE = (95, 100), (150, 155)


def a_operand(seed, M, K, chunk):
    """Codes and E8M0 scale bytes ([M][K/chunk]) for A, banded by row index mod 4."""
    rng = np.random.default_rng(seed)
    a = synth.random_codes(seed + 1, (M, K), 0)
    band = np.arange(M) % 4
    a[band == 2] &= 0x7F
    sparse = np.flatnonzero(band == 3)
    a[sparse] = 0
    for i in sparse:
        ks = rng.choice(K, 2, replace=False)
        a[i, ks] = synth.random_codes(seed + 2 + int(i), (2,), 0)
    sa = np.empty((M, K // chunk), np.uint8)
    for j, (lo, hi) in enumerate(A_BANDS):
        rows = band == j
        sa[rows] = rng.integers(lo, hi + 1, size=(int(rows.sum()), K // chunk), dtype=np.uint8)
    return a, sa


def b_scale_bytes(seed, n_col_groups, n_k):
    """[column group][K group] bytes: small scales on even groups, large on odd."""
    rng = np.random.default_rng(seed)
    small = rng.integers(B_SMALL[0], B_SMALL[1] + 1, size=(n_col_groups, n_k), dtype=np.uint8)
    large = rng.integers(B_LARGE[0], B_LARGE[1] + 1, size=(n_col_groups, n_k), dtype=np.uint8)
    return np.where((np.arange(n_col_groups) % 2 == 0)[:, None], small, large)


def rne_bits(y32):
    """fp32 CUDA tensor -> int16 bits of its nearest-even bf16 (rounded on the CPU)."""
    return y32.cpu().to(torch.bfloat16).view(torch.int16)


def check_rne(y32, y16, what, coverage=False):
    """coverage: also require each class of result above to occur (on large outputs;
    the finite values that round to infinity lie in a window 2^-8 of an octave wide)."""
    got, want = y16.cpu().view(torch.int16), rne_bits(y32)
    if not torch.equal(got, want):
        bad = (got != want).nonzero()[:8].tolist()
        v = y32.cpu()
        raise AssertionError("%s: bf16 output differs from RNE(fp32 output) at %s (fp32 bits %s)" % (
            what, bad, [hex(int(v[i, j].view(torch.int32))) for i, j in bad]))
    assert not torch.isnan(y32).any()
    if coverage:
        bits = y32.cpu().view(torch.int32).numpy().view(np.uint32)
        mag = bits & 0x7FFFFFFF
        low = bits & 0x1FFFF
        assert np.count_nonzero((mag > 0) & (mag < 0x00800000)) > 0, "no subnormal result"
        assert np.count_nonzero(mag == 0x7F800000) > 0, "no fp32 overflow"
        assert np.count_nonzero((mag >= 0x7F7F8000) & (mag < 0x7F800000)) > 0, "no finite result rounding to inf"
        assert np.count_nonzero(low == 0x8000) > 0 and np.count_nonzero(low == 0x18000) > 0, "no halfway case"


@pytest.mark.parametrize("b_layout", [mx.B_NK, mx.B_KN])
@pytest.mark.parametrize("shape", SHAPES)
def test_block_scaled(b_layout, shape):
    M, N, K = shape
    a, sa = a_operand(9100 + M, M, K, 128)
    b_nk = synth.random_codes(9101, (N, K), 0) & 0x7F
    sb_nk = b_scale_bytes(9102, (N + 127) // 128, K // 128)
    if b_layout == mx.B_NK:
        b, sb = dev(b_nk), dev(sb_nk)
    else:
        b, sb = dev(np.ascontiguousarray(b_nk.T)), dev(np.ascontiguousarray(sb_nk.T))
    args = (dev(a), dev(sa), mx.E4M3, b, sb, mx.E4M3, b_layout, mx.SCALE_BLOCK128)
    y32 = mx.block_scaled_gemm(*args, out_dtype=torch.float32)
    y16 = mx.block_scaled_gemm(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check_rne(y32, y16, "block-scaled %s layout %d" % (shape, b_layout), coverage=M * N >= 1 << 24)


@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[2]])
def test_mx(shape):
    M, N, K = shape
    a, sa = a_operand(9200 + M, M, K, 32)
    b = synth.random_codes(9201, (N, K), 0) & 0x7F
    sb = np.repeat(b_scale_bytes(9202, (N + 127) // 128, K // 32), 128, axis=0)[:N]
    args = (dev(a), dev(sa), mx.E4M3, dev(b), dev(np.ascontiguousarray(sb)), mx.E4M3)
    y32 = mx.mx_scaled_gemm(*args, out_dtype=torch.float32)
    y16 = mx.mx_scaled_gemm(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check_rne(y32, y16, "MX %s" % (shape,), coverage=M * N >= 1 << 24)


@pytest.mark.parametrize("shape", [SHAPES[0], (2048, 2048, 512)])
def test_f32s(shape):
    """fp32 scales: powers of two from the same bands, the subnormal band's raised
    so that fl(sa * sb) stays a normal number (its results are still partly
    subnormal)."""
    M, N, K = shape
    a, sa = a_operand(9300 + M, M, K, 128)
    sa = np.where(sa < 64, sa + 30, sa)
    b = synth.random_codes(9301, (N, K), 0) & 0x7F
    sb = b_scale_bytes(9302, (N + 127) // 128, K // 128)
    to_f32 = lambda e: np.ldexp(1.0, e.astype(np.int32) - 127).astype(np.float32)
    args = (dev(a), dev(to_f32(sa)), mx.E4M3, dev(b), dev(to_f32(sb)), mx.E4M3)
    y32 = mx.gemm_f32s(*args, out_dtype=torch.float32)
    y16 = mx.gemm_f32s(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check_rne(y32, y16, "fp32 scales %s" % (shape,))
