// gaussws.hip -- GaussWS weight sampling for gfx950 ["Gaussian Weight
// Sampling for Scalable, Efficient and Stable Pseudo-Quantization Training",
// review page, "What carries the argument"]: the sampled weight
// w_hat = w + R * max_bl(|w|) * 2^(1 - b_t), per 32x32 block with its own
// bitwidth b_t, cast to BF16, where R is the nearest integer to N(0,1)/2.
//
// R is drawn by its definition (the page's bitwise approximation is not
// printed): |R| = 0, 1, 2 as |Z| < 1, 1 <= |Z| < 3, |Z| >= 3, decided on 31
// uniform bits against the normal's quantiles, the 32nd bit the sign.  The
// bits come from the counter-based Philox4x64-10 generator (Salmon, Moraes,
// Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11): key
// (seed, stream), counter (col / 8, row, 0, 0); the four 64-bit outputs give
// the 32-bit words of columns col .. col + 7 (low half first).  So every
// element's noise depends only on (seed, stream, row, col), whatever the
// launch shape.
//
// One workgroup per 32 rows x 256 columns: eight 32x32 blocks, one per
// 32-lane half wave.  A lane holds 4 rows x 8 columns (one Philox call per
// row), the block maximum reduces over its 32 lanes, and each row of 8
// outputs goes out as one 16-byte store.  The input is read once.
#include "device_common.hpp"
#include "launch.hpp"

namespace mxfp8 {

namespace gaussws_detail {

constexpr int kThreads = 256;

// x * M as a 128-bit product (hi, lo) from 32-bit halves (schoolbook, three
// partial sums that cannot overflow 64 bits): four 32 x 32 + 64 -> 64-bit
// multiply-adds.  Written out, it compiles to about half the instructions of
// the generic 64-bit high and low products.
template <uint64_t M>
__device__ __forceinline__ void mul_64x64(uint64_t x, uint64_t& hi, uint64_t& lo) {
  constexpr uint32_t ml = (uint32_t)M, mh = (uint32_t)(M >> 32);
  const uint32_t xl = (uint32_t)x, xh = (uint32_t)(x >> 32);
  const uint64_t t0 = (uint64_t)xl * ml;                    // bits 0 .. 63
  const uint64_t t1 = (uint64_t)xh * ml + (t0 >> 32);       // bits 32 .. 95
  const uint64_t t2 = (uint64_t)xl * mh + (uint32_t)t1;     // bits 32 .. 95
  hi = (uint64_t)xh * mh + (t1 >> 32) + (t2 >> 32);
  lo = (t2 << 32) | (uint32_t)t0;
}

// Philox4x64-10: ten rounds of two 64 x 64 -> 128-bit products, key bumped by
// the Weyl increments after each round.
struct U64x4 {
  uint64_t v[4];
};
__device__ __forceinline__ U64x4 philox4x64_10(uint64_t x0, uint64_t x1, uint64_t x2, uint64_t x3, uint64_t k0,
                                               uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    uint64_t hi0, lo0, hi1, lo1;
    mul_64x64<M0>(x0, hi0, lo0);
    mul_64x64<M1>(x2, hi1, lo1);
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  return U64x4{{x0, x1, x2, x3}};
}

// |R| thresholds on 31 uniform bits: round(erf(1 / sqrt 2) * 2^31) and
// round(erf(3 / sqrt 2) * 2^31), i.e. P(|Z| < 1) and P(|Z| < 3).
constexpr uint32_t kR1 = 1466064521u, kR2 = 2141685880u;

__device__ __forceinline__ float rounded_normal(uint32_t u) {
  const uint32_t m = u & 0x7FFFFFFFu;
  const float mag = m < kR1 ? 0.0f : (m < kR2 ? 1.0f : 2.0f);
  return (u >> 31) ? -mag : mag;
}

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest-even bf16, packed (lo in bits 0-15):
// one v_cvt_pk_bf16_f32 (the default round mode is nearest-even; subnormals
// are kept; a NaN stays a NaN).
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2bf));
}

template <typename InT, bool NT>
__global__ __launch_bounds__(kThreads) void gaussws_kernel(const InT* __restrict__ w, uint32_t rows, uint32_t cols,
                                                           int64_t ldw, const int8_t* __restrict__ bt, uint32_t nbc,
                                                           uint64_t seed, uint64_t stream_id,
                                                           uint16_t* __restrict__ out, int64_t ldo) {
  const uint32_t tid = threadIdx.x;
  const uint32_t gx = (cols + 255) >> 8;   // 1-D grid: workgroup b is strip (b % gx, b / gx)
  const uint32_t by = blockIdx.x / gx, bx = blockIdx.x - by * gx;
  const uint32_t j = tid >> 5;             // block of the strip
  const uint32_t cc = tid & 3;             // 8-column chunk in the block
  const uint32_t rg = (tid & 31) >> 2;     // 4-row group in the block
  const uint32_t r0 = by * 32 + rg * 4;
  const uint32_t col = bx * 256 + j * 32 + cc * 8;
  const bool cact = col < cols;            // cols % 8 == 0: a chunk is wholly in or out
  float f[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (cact && r0 + i < rows) load8<NT>(w + (int64_t)(r0 + i) * ldw + col, f[i]);
    else
#pragma unroll
      for (int k = 0; k < 8; ++k) f[i][k] = 0.0f;
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 8; ++k) m = max(m, abs_bits(f[i][k]));
  m = max_row16(m);
  const uint32_t o = (uint32_t)__shfl_xor((int)m, 16);
  m = m > o ? m : o;  // the 32 lanes of this block
  const uint32_t bj = (bx * 256 + j * 32) >> 5;
  const int b = bj < nbc ? (int)bt[(int64_t)by * nbc + bj] : 0;
  const float scale = ldexpf(__uint_as_float(m), 1 - b);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t r = r0 + i;
    if (!cact || r >= rows) continue;
    const U64x4 u = philox4x64_10(col >> 3, r, 0, 0, seed, stream_id);
    uint32_t h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = f[i][2 * q] + rounded_normal((uint32_t)u.v[q]) * scale;
      const float hi = f[i][2 * q + 1] + rounded_normal((uint32_t)(u.v[q] >> 32)) * scale;
      h[q] = bf16x2_rne(lo, hi);
    }
    *reinterpret_cast<uint4*>(out + (int64_t)r * ldo + col) = make_uint4(h[0], h[1], h[2], h[3]);
  }
}

}  // namespace gaussws_detail

using namespace gaussws_detail;

void launch_gaussws(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw, const int8_t* bt,
                    uint64_t seed, uint64_t stream_id, uint16_t* out, int64_t ldo, hipStream_t stream) {
  const uint32_t nbc = (uint32_t)((cols + 31) / 32);
  const dim3 grid((uint32_t)((cols + 255) / 256) * (uint32_t)((rows + 31) / 32));
  if (dtype == 1) {
    const auto kern = stream_loads(rows, cols, 2) ? gaussws_kernel<uint16_t, true> : gaussws_kernel<uint16_t, false>;
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, stream, (const uint16_t*)w, (uint32_t)rows, (uint32_t)cols,
                       ldw, bt, nbc, seed, stream_id, out, ldo);
  } else {
    const auto kern = stream_loads(rows, cols, 4) ? gaussws_kernel<float, true> : gaussws_kernel<float, false>;
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, stream, (const float*)w, (uint32_t)rows, (uint32_t)cols, ldw,
                       bt, nbc, seed, stream_id, out, ldo);
  }
}

}  // namespace mxfp8
