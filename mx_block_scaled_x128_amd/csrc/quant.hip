// quant.hip -- HBM-streaming FP8 quantizers for gfx950.
//
// Token-wise 1x128 groups (activations / gradients) and 128x128 tiles
// (weights) with round-up power-of-two UE8M0 scales ["A Comprehensive FP8
// Training Recipe for Reasoning-Enhanced Language Models", "What carries the
// argument", Figs. 1-2]; 32-element MX blocks with the OCP floor rule and the
// clamp counter ["Characterization and Mitigation of Training Instabilities in
// Microscaling Formats", "What carries the argument", Fig. 5].
//
// Every kernel reads its input once (16-byte vector loads, 8 elements per
// lane), reduces amax with DPP inside the wavefront (LDS only where a group
// spans waves), and writes packed codes (8 bytes per lane) with ordinary
// stores, which leave them in the last-level cache for the GEMM.  NT (a
// template parameter, chosen per launch by stream_loads): non-temporal input
// loads, for inputs of 64 MiB or more.
#include "device_common.hpp"
#include "launch.hpp"

namespace mxfp8 {

namespace quant_detail {

constexpr int kThreads = 256;
// quant_col_t_kernel and quant_dual_kernel: 8 waves per 128x128 tile, 4
// tokens x 8 channels per thread (measured 4-6 % and 7-10 % faster than 4
// waves with 8 tokens each).
constexpr int kColThreads = 512;
// quant_block_kernel: 8 waves per 128x128 tile, 4 rows x 8 columns per
// thread (measured 2-5 % faster than 4 waves with 8 rows each).
constexpr int kBlockThreads = 512;
static_assert(kBlockThreads == 512, "quant_block_kernel's reduction reads 8 wave maxima");
constexpr uint32_t kMaxBlocks = 256 * 8;  // 8 workgroups per CU, grid-stride beyond that

// Tile kernels run on 1-D grids (a 2-D grid's y extent is limited to 65535):
// workgroup b is tile (b % gx, b / gx) of a gx-wide tile grid, x fastest.
struct TileXY {
  uint32_t x, y;
};
__device__ __forceinline__ TileXY tile_xy(uint32_t gx) {
  const uint32_t y = blockIdx.x / gx;
  return TileXY{blockIdx.x - y * gx, y};
}

__device__ __forceinline__ void zero8(float (&f)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = 0.0f;
}

template <int FMT>
__device__ __forceinline__ uint2 codes8(const float (&f)[8], float sc) {
  uint2 o;
  o.x = cvt4<FMT>(f[0] * sc, f[1] * sc, f[2] * sc, f[3] * sc);
  o.y = cvt4<FMT>(f[4] * sc, f[5] * sc, f[6] * sc, f[7] * sc);
  return o;
}

// Eight codes under an fp32 scale: the fp32 quotient x / s (IEEE division),
// clamped to +-fmax (the saturation of the cast; quotients can exceed fmax by
// the rounding of s), then the hardware RNE cast.
template <int FMT>
__device__ __forceinline__ uint32_t cvt4_div(float a, float b, float c, float d, float s) {
  constexpr float fmax = FmtInfo<FMT>::fmax;
  return cvt4<FMT>(__builtin_amdgcn_fmed3f(a / s, -fmax, fmax), __builtin_amdgcn_fmed3f(b / s, -fmax, fmax),
                   __builtin_amdgcn_fmed3f(c / s, -fmax, fmax), __builtin_amdgcn_fmed3f(d / s, -fmax, fmax));
}
template <int FMT>
__device__ __forceinline__ uint2 codes8_div(const float (&f)[8], float s) {
  uint2 o;
  o.x = cvt4_div<FMT>(f[0], f[1], f[2], f[3], s);
  o.y = cvt4_div<FMT>(f[4], f[5], f[6], f[7], s);
  return o;
}

// Row pitch of the transposed code tiles in LDS (bytes); see quant_col_t_kernel.
constexpr int kColPitch = 136;

// A 128 x 128-byte tile of codes in LDS in the layout of the output (rows of
// 128 bytes, no padding): the 8-byte chunk c of row r sits in 16-byte slot
// (c >> 1) ^ ((r >> 3) & 7), half c & 1.  The writers (quant_dual_kernel: a
// lane's 4 rows are 4 apart, 16 lanes cover 8 row groups and 2 chunks;
// quant_block_dual_kernel: 8 rows 8 apart) put one chunk of many rows at once,
// and the XOR spreads those rows' chunks over different slots; readers take
// whole 16-byte slots.  Every store instruction then writes 8 full 128-byte
// rows instead of 64-byte halves of lines from two different waves.
__device__ __forceinline__ uint32_t row_tile_offset(uint32_t r, uint32_t c) {
  return r * 128 + ((((c >> 1) ^ ((r >> 3) & 7)) << 4) | ((c & 1) << 3));
}
template <int NT = kThreads>
__device__ __forceinline__ void store_row_tile(const uint8_t* rtile, uint8_t* __restrict__ q, int64_t ldq,
                                               uint32_t r0, uint32_t c0, uint32_t rows, uint32_t cols,
                                               uint32_t tid) {
#pragma unroll
  for (int rep = 0; rep < 1024 / NT; ++rep) {
    const uint32_t idx = rep * NT + tid;
    const uint32_t r = idx >> 3, p = idx & 7;
    if (r0 + r < rows && c0 + p * 16 < cols) {
      const uint4 v = *reinterpret_cast<const uint4*>(rtile + r * 128 + ((p ^ ((r >> 3) & 7)) << 4));
      store_codes(q + (int64_t)(r0 + r) * ldq + c0 + p * 16, v);
    }
  }
}
// The transposed tile of quant_col_t_kernel (rows of kColPitch bytes) out to
// qt [cols][ldqt]: 16 bytes per lane, 8 lanes per 128-token row.
template <int NT = kThreads>
__device__ __forceinline__ void store_tile_t(const uint8_t* tile, uint8_t* __restrict__ qt, int64_t ldqt,
                                             uint32_t c0, uint32_t t0, uint32_t cols, uint32_t rows,
                                             uint32_t tid) {
#pragma unroll
  for (int rep = 0; rep < 1024 / NT; ++rep) {
    const uint32_t idx = rep * NT + tid;
    const uint32_t ch = idx >> 3, ck = idx & 7;
    if (c0 + ch < cols && t0 + ck * 16 < rows) {
      const uint2 a = *reinterpret_cast<const uint2*>(tile + ch * kColPitch + ck * 16);
      const uint2 b = *reinterpret_cast<const uint2*>(tile + ch * kColPitch + ck * 16 + 8);
      store_codes(qt + (int64_t)(c0 + ch) * ldqt + t0 + ck * 16, make_uint4(a.x, a.y, b.x, b.y));
    }
  }
}

// ---------------------------------------------------------------------------
// 1x128 groups along rows.  A wavefront handles "items" of 4 consecutive
// groups of one row: 16 lanes per group, 8 elements per lane.  Items are
// wave-uniform, so the row / column split runs on the scalar unit.
// ---------------------------------------------------------------------------
// F32S: fp32 scales (scale_f32, codes8_div) instead of E8M0 bytes; s then
// points to floats.
template <typename InT, int FMT, int U, bool F32S, bool NT>
__global__ __launch_bounds__(kThreads) void quant_row_kernel(
    const InT* __restrict__ x, uint32_t cols, int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
    void* __restrict__ s, uint32_t ngroups, uint32_t ipr, uint32_t total_items) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t sub = lane & 15;
  const uint32_t slot = lane >> 4;
  // Known uniform: the item index math (row = item / items per row, addresses)
  // then runs on the scalar unit.
  const uint32_t wave = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t nwaves = gridDim.x * (kThreads / 64);
  for (uint32_t it = wave * U; it < total_items; it += nwaves * U) {
    float f[U][8];
    uint32_t row[U], grp[U];
    bool act[U], gvalid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t item = it + u;
      const uint32_t r = item / ipr;
      const uint32_t g = (item - r * ipr) * 4 + slot;
      const uint32_t c = g * 128 + sub * 8;
      row[u] = r;
      grp[u] = g;
      gvalid[u] = item < total_items && g < ngroups;
      act[u] = gvalid[u] && c < cols;
      if (act[u]) load8<NT>(x + (int64_t)r * ldx + c, f[u]);
      else zero8(f[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = max(m, abs_bits(f[u][j]));
      m = max_row16(m);
      if constexpr (F32S) {
        const float sf = scale_f32<FMT>(m);
        if (act[u])
          store_codes(q + (int64_t)row[u] * ldq + grp[u] * 128 + sub * 8, codes8_div<FMT>(f[u], sf));
        if (sub == 0 && gvalid[u]) static_cast<float*>(s)[(int64_t)row[u] * ngroups + grp[u]] = sf;
      } else {
        const int e = scale_exp_ceil<FMT>(m);
        const float sc = pow2_neg(e);
        if (act[u])
          store_codes(q + (int64_t)row[u] * ldq + grp[u] * 128 + sub * 8, codes8<FMT>(f[u], sc));
        if (sub == 0 && gvalid[u]) static_cast<uint8_t*>(s)[(int64_t)row[u] * ngroups + grp[u]] = (uint8_t)(e + 127);
      }
    }
  }
}

// Raw input of 8 elements (bf16: one 16-byte word; fp32: two), converted
// when used, so a prefetched tile costs 4 (bf16) or 8 registers per row.
template <typename InT> struct Raw8;
template <> struct Raw8<uint16_t> { nt_u32x4 v; };
template <> struct Raw8<float> { nt_f32x4 a, b; };
template <bool NT>
__device__ __forceinline__ void raw_load(const uint16_t* p, Raw8<uint16_t>& r) {
  r.v = NT ? __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p)) : *reinterpret_cast<const nt_u32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ void raw_load(const float* p, Raw8<float>& r) {
  r.a = NT ? __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p)) : *reinterpret_cast<const nt_f32x4*>(p);
  r.b = NT ? __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p + 4))
           : *reinterpret_cast<const nt_f32x4*>(p + 4);
}
__device__ __forceinline__ void raw_zero(Raw8<uint16_t>& r) { r.v = nt_u32x4{0, 0, 0, 0}; }
__device__ __forceinline__ void raw_zero(Raw8<float>& r) { r.a = nt_f32x4{0, 0, 0, 0}; r.b = r.a; }
__device__ __forceinline__ void raw_f8(const Raw8<uint16_t>& r, float (&f)[8]) {
  f[0] = bf16_lo(r.v.x); f[1] = bf16_hi(r.v.x); f[2] = bf16_lo(r.v.y); f[3] = bf16_hi(r.v.y);
  f[4] = bf16_lo(r.v.z); f[5] = bf16_hi(r.v.z); f[6] = bf16_lo(r.v.w); f[7] = bf16_hi(r.v.w);
}
// Max of |x| bits over the 8 elements, from the raw words.
__device__ __forceinline__ uint32_t raw_absmax(const Raw8<uint16_t>& r) {
  const uint32_t a = max((r.v.x << 16) & 0x7FFFFFFFu, r.v.x & 0x7FFF0000u);
  const uint32_t b = max((r.v.y << 16) & 0x7FFFFFFFu, r.v.y & 0x7FFF0000u);
  const uint32_t c = max((r.v.z << 16) & 0x7FFFFFFFu, r.v.z & 0x7FFF0000u);
  const uint32_t d = max((r.v.w << 16) & 0x7FFFFFFFu, r.v.w & 0x7FFF0000u);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t raw_absmax(const Raw8<float>& r) {
  float f[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = max(m, abs_bits(f[j]));
  return m;
}
__device__ __forceinline__ void raw_f8(const Raw8<float>& r, float (&f)[8]) {
  f[0] = r.a.x; f[1] = r.a.y; f[2] = r.a.z; f[3] = r.a.w;
  f[4] = r.b.x; f[5] = r.b.y; f[6] = r.b.z; f[7] = r.b.w;
}

// Element j (0..7; a compile-time constant after unrolling) of raw words.
__device__ __forceinline__ float raw_elem(const Raw8<uint16_t>& r, int j) {
  const uint32_t wd = j < 2 ? r.v.x : j < 4 ? r.v.y : j < 6 ? r.v.z : r.v.w;
  return (j & 1) ? bf16_hi(wd) : bf16_lo(wd);
}
__device__ __forceinline__ float raw_elem(const Raw8<float>& r, int j) {
  return j < 4 ? r.a[j] : r.b[j - 4];
}
// ---------------------------------------------------------------------------
// 128-token groups down columns, codes written transposed (token axis
// contiguous).  One workgroup of 8 waves per 128 tokens x 128 channels tile:
// each thread holds 4 tokens x 8 channels in registers; column maxima reduce
// over the 8 lanes of a wave that share a channel chunk (DPP), then over the
// four waves that cover the tile's token quarters (LDS).  Codes are transposed through an
// LDS tile whose rows are padded to 136 bytes (16-byte aligned rows for the
// stores; each thread writes its 4 tokens' codes of a channel as 4 bytes).
// ---------------------------------------------------------------------------

template <typename InT, int FMT, bool F32S, bool NT>
__global__ __launch_bounds__(kColThreads) void quant_col_t_kernel(
    const InT* __restrict__ x, uint32_t rows, uint32_t cols, int64_t ldx, uint8_t* __restrict__ qt,
    int64_t ldq, void* __restrict__ st, uint32_t ngt) {
  __shared__ uint32_t red[4][128];
  __shared__ int exps[128];  // exponents, or with F32S the fp32 scales' bits
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * kColPitch];
  const uint32_t tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t tr = (lane & 7) + 8 * (w & 3);   // token chunk: tokens tr*4 .. tr*4+3
  const uint32_t tc = (lane >> 3) + 8 * (w >> 2); // channel chunk: channels tc*8 .. tc*8+7
  const TileXY b = tile_xy((cols + 127) >> 7);
  const uint32_t c0 = b.x * 128, t0 = b.y * 128;
  const bool cact = c0 + tc * 8 < cols;
  // The input stays in its raw words (bf16: 4 registers per token), each
  // element converted where it is used: holding 32 fp32 values instead made
  // the kernel 4 % slower (11 % with fp32 scales).
  Raw8<InT> rr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t r = t0 + tr * 4 + i;
    if (cact && r < rows) raw_load<NT>(x + (int64_t)r * ldx + c0 + tc * 8, rr[i]);
    else raw_zero(rr[i]);
  }
  uint32_t m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    m[j] = max_oct(max(max(abs_bits(raw_elem(rr[0], j)), abs_bits(raw_elem(rr[1], j))),
                       max(abs_bits(raw_elem(rr[2], j)), abs_bits(raw_elem(rr[3], j)))));
  if ((lane & 7) == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) red[w & 3][tc * 8 + j] = m[j];
  }
  __syncthreads();
  if (tid < 128) {
    const uint32_t a = max(max(red[0][tid], red[1][tid]), max(red[2][tid], red[3][tid]));
    if constexpr (F32S) {
      const float sf = scale_f32<FMT>(a);
      exps[tid] = __float_as_int(sf);
      if (c0 + tid < cols) static_cast<float*>(st)[(int64_t)(c0 + tid) * ngt + b.y] = sf;
    } else {
      const int e = scale_exp_ceil<FMT>(a);
      exps[tid] = e;
      if (c0 + tid < cols) static_cast<uint8_t*>(st)[(int64_t)(c0 + tid) * ngt + b.y] = (uint8_t)(e + 127);
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float f0 = raw_elem(rr[0], j), f1 = raw_elem(rr[1], j), f2 = raw_elem(rr[2], j),
                f3 = raw_elem(rr[3], j);  // tokens 0..3 of channel j
    uint32_t o;
    if constexpr (F32S) {
      const float sf = __int_as_float(exps[tc * 8 + j]);
      o = cvt4_div<FMT>(f0, f1, f2, f3, sf);
    } else {
      const float sc = pow2_neg(exps[tc * 8 + j]);
      o = cvt4<FMT>(f0 * sc, f1 * sc, f2 * sc, f3 * sc);
    }
    *reinterpret_cast<uint32_t*>(tile + (tc * 8 + j) * kColPitch + tr * 4) = o;
  }
  __syncthreads();
  store_tile_t<kColThreads>(tile, qt, ldq, c0, t0, cols, rows, tid);
}

// ---------------------------------------------------------------------------
// Both orientations of the token-wise quantization from one read of x: the
// 1x128 row groups (codes in x's layout) and the 128-token column groups
// (codes transposed).  The tile and thread layout are those of
// quant_col_t_kernel; a tile's 128 channels are exactly one row group of each
// of its 128 tokens (tiles start on multiples of 128), so each token's row
// maximum reduces over the 8 lanes of a wave that share its token chunk
// (stride-8 lanes) and then over the two waves that cover the tile's channel
// halves (LDS).  Both code sets are staged in LDS and stored as whole rows.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t max_stride8(uint32_t v) {
  v = dpp_max<DPP_ROW_ROR8>(v);
  uint32_t o = (uint32_t)__shfl_xor((int)v, 16);
  v = v > o ? v : o;
  o = (uint32_t)__shfl_xor((int)v, 32);
  return v > o ? v : o;
}

template <typename InT, int FMT, bool NT>
__global__ __launch_bounds__(kColThreads) void quant_dual_kernel(
    const InT* __restrict__ x, uint32_t rows, uint32_t cols, int64_t ldx, uint8_t* __restrict__ q,
    int64_t ldq, uint8_t* __restrict__ s, uint8_t* __restrict__ qt, int64_t ldqt, uint8_t* __restrict__ st,
    uint32_t ngc, uint32_t ngt) {
  __shared__ uint32_t red[4][128];   // column maxima per token quarter
  __shared__ uint32_t rred[2][128];  // row maxima per channel half
  __shared__ int exps[128], rexps[128];
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * kColPitch];
  __shared__ __attribute__((aligned(16))) uint8_t rtile[128 * 128];
  const uint32_t tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t tr = (lane & 7) + 8 * (w & 3);   // token chunk: tokens tr*4 .. tr*4+3
  const uint32_t tc = (lane >> 3) + 8 * (w >> 2); // channel chunk: channels tc*8 .. tc*8+7
  const TileXY b = tile_xy(ngc);
  const uint32_t c0 = b.x * 128, t0 = b.y * 128;
  const bool cact = c0 + tc * 8 < cols;
  Raw8<InT> rr[4];  // [token], raw words, converted where used
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t r = t0 + tr * 4 + i;
    if (cact && r < rows) raw_load<NT>(x + (int64_t)r * ldx + c0 + tc * 8, rr[i]);
    else raw_zero(rr[i]);
  }
  uint32_t m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    m[j] = max_oct(max(max(abs_bits(raw_elem(rr[0], j)), abs_bits(raw_elem(rr[1], j))),
                       max(abs_bits(raw_elem(rr[2], j)), abs_bits(raw_elem(rr[3], j)))));
  if ((lane & 7) == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) red[w & 3][tc * 8 + j] = m[j];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) m[i] = max_stride8(raw_absmax(rr[i]));
  if ((lane >> 3) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) rred[w >> 2][tr * 4 + i] = m[i];
  }
  __syncthreads();
  if (tid < 128) {
    const uint32_t a = max(max(red[0][tid], red[1][tid]), max(red[2][tid], red[3][tid]));
    const int e = scale_exp_ceil<FMT>(a);
    exps[tid] = e;
    if (c0 + tid < cols) st[(int64_t)(c0 + tid) * ngt + b.y] = (uint8_t)(e + 127);
  } else if (tid < 256) {
    const uint32_t t = tid - 128;
    const uint32_t a = max(rred[0][t], rred[1][t]);
    const int e = scale_exp_ceil<FMT>(a);
    rexps[t] = e;
    if (t0 + t < rows) s[(int64_t)(t0 + t) * ngc + b.x] = (uint8_t)(e + 127);
  }
  __syncthreads();
  // Column codes into the transposed tile; row codes into the row tile.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float sc = pow2_neg(exps[tc * 8 + j]);
    *reinterpret_cast<uint32_t*>(tile + (tc * 8 + j) * kColPitch + tr * 4) =
        cvt4<FMT>(raw_elem(rr[0], j) * sc, raw_elem(rr[1], j) * sc, raw_elem(rr[2], j) * sc,
                  raw_elem(rr[3], j) * sc);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f[8];
    raw_f8(rr[i], f);
    *reinterpret_cast<uint2*>(rtile + row_tile_offset(tr * 4 + i, tc)) = codes8<FMT>(f, pow2_neg(rexps[tr * 4 + i]));
  }
  __syncthreads();
  store_tile_t<kColThreads>(tile, qt, ldqt, c0, t0, cols, rows, tid);
  store_row_tile<kColThreads>(rtile, q, ldq, t0, c0, rows, cols, tid);
}

// ---------------------------------------------------------------------------
// 128x128 tiles with both the codes and their transpose (one scale per tile,
// so the transposed codes are the same bytes): thread layout of
// quant_col_t_kernel, amax over the whole tile, both code sets staged in LDS
// (the padded transposed tile and the swizzled row tile).
// ---------------------------------------------------------------------------
template <typename InT, int FMT, bool NT>
__global__ __launch_bounds__(kThreads) void quant_block_dual_kernel(
    const InT* __restrict__ w, uint32_t rows, uint32_t cols, int64_t ldw, uint8_t* __restrict__ q,
    int64_t ldq, uint8_t* __restrict__ s, uint8_t* __restrict__ qt, int64_t ldqt, uint8_t* __restrict__ st,
    uint32_t nbc, uint32_t nbr) {
  __shared__ uint32_t red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * kColPitch];
  __shared__ __attribute__((aligned(16))) uint8_t rtile[128 * 128];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t tr = (lane & 7) + 8 * (wv & 1);   // row chunk: rows tr*8 .. tr*8+7
  const uint32_t tc = (lane >> 3) + 8 * (wv >> 1); // column chunk: columns tc*8 .. tc*8+7
  const TileXY b = tile_xy(nbc);
  const uint32_t c0 = b.x * 128, r0 = b.y * 128;
  const bool cact = c0 + tc * 8 < cols;
  Raw8<InT> rr[8];  // [row], raw words, converted where used
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t r = r0 + tr * 8 + i;
    if (cact && r < rows) raw_load<NT>(w + (int64_t)r * ldw + c0 + tc * 8, rr[i]);
    else raw_zero(rr[i]);
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, raw_absmax(rr[i]));
  m = max_wave(m);
  if (lane == 0) red[wv] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  const int e = scale_exp_ceil<FMT>(m);
  const float sc = pow2_neg(e);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint2 o;
    o.x = cvt4<FMT>(raw_elem(rr[0], j) * sc, raw_elem(rr[1], j) * sc, raw_elem(rr[2], j) * sc,
                    raw_elem(rr[3], j) * sc);
    o.y = cvt4<FMT>(raw_elem(rr[4], j) * sc, raw_elem(rr[5], j) * sc, raw_elem(rr[6], j) * sc,
                    raw_elem(rr[7], j) * sc);
    *reinterpret_cast<uint2*>(tile + (tc * 8 + j) * kColPitch + tr * 8) = o;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float f[8];
    raw_f8(rr[i], f);
    *reinterpret_cast<uint2*>(rtile + row_tile_offset(tr * 8 + i, tc)) = codes8<FMT>(f, sc);
  }
  if (tid == 0) {
    s[(int64_t)b.y * nbc + b.x] = (uint8_t)(e + 127);
    st[(int64_t)b.x * nbr + b.y] = (uint8_t)(e + 127);
  }
  __syncthreads();
  store_tile_t(tile, qt, ldqt, c0, r0, cols, rows, tid);
  store_row_tile(rtile, q, ldq, r0, c0, rows, cols, tid);
}

// ---------------------------------------------------------------------------
// 128x128 tiles.  One workgroup per tile, the whole tile held in registers
// (4 rows x 8 columns per thread, 8 wavefronts), amax by DPP + cross-lane
// shuffles inside each wavefront and 8 values through LDS across wavefronts;
// then one pass of casts and 8-byte stores.  Input is read from HBM exactly
// once.
// ---------------------------------------------------------------------------
// PIPE: each workgroup takes tiles blockIdx.x, + gridDim.x, ... and loads
// its next tile before the current one's reduction, barrier and stores, so
// its loads stay in flight across them (72 registers: 7 waves per SIMD,
// three workgroups per CU).  Otherwise one tile per workgroup (four
// workgroups per CU): inputs of at most one round of tiles, and the
// fp32-scale variant, whose divisions made the pipelined form slower.
template <typename InT, int FMT, bool F32S, bool NT, bool PIPE>
__global__ __launch_bounds__(kBlockThreads) void quant_block_kernel(
    const InT* __restrict__ w, uint32_t rows, uint32_t cols, int64_t ldw, uint8_t* __restrict__ q,
    int64_t ldq, void* __restrict__ s, uint32_t nbc, uint32_t ntiles) {
  __shared__ uint32_t red[2][kBlockThreads / 64];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t tc = lane & 15;               // column chunk: columns tc*8 .. tc*8+7
  const uint32_t tr = (lane >> 4) + 4 * wv;    // row chunk: rows tr*4 .. tr*4+3
  auto load_tile = [&](uint32_t t, Raw8<InT> (&rr)[4]) __attribute__((always_inline)) {
    const uint32_t by = t / nbc, bx = t - by * nbc;
    const uint32_t r0 = by * 128, c0 = bx * 128;
    const bool cact = c0 + tc * 8 < cols;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t r = r0 + tr * 4 + i;
      if (cact && r < rows) raw_load<NT>(w + (int64_t)r * ldw + c0 + tc * 8, rr[i]);
      else raw_zero(rr[i]);
    }
  };
  auto process = [&](uint32_t t, const Raw8<InT> (&rr)[4], int par) __attribute__((always_inline)) {
    const uint32_t by = t / nbc, bx = t - by * nbc;
    const uint32_t r0 = by * 128, c0 = bx * 128;
    const bool cact = c0 + tc * 8 < cols;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, raw_absmax(rr[i]));
    m = max_wave(m);
    if (lane == 0) red[par][wv] = m;
    __syncthreads();
    m = max(max(max(red[par][0], red[par][1]), max(red[par][2], red[par][3])),
            max(max(red[par][4], red[par][5]), max(red[par][6], red[par][7])));
    if constexpr (F32S) {
      const float sf = scale_f32<FMT>(m);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t r = r0 + tr * 4 + i;
        float f[8];
        raw_f8(rr[i], f);
        if (cact && r < rows) store_codes(q + (int64_t)r * ldq + c0 + tc * 8, codes8_div<FMT>(f, sf));
      }
      if (tid == 0) static_cast<float*>(s)[(int64_t)by * nbc + bx] = sf;
    } else {
      const int e = scale_exp_ceil<FMT>(m);
      const float sc = pow2_neg(e);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t r = r0 + tr * 4 + i;
        float f[8];
        raw_f8(rr[i], f);
        if (cact && r < rows) store_codes(q + (int64_t)r * ldq + c0 + tc * 8, codes8<FMT>(f, sc));
      }
      if (tid == 0) static_cast<uint8_t*>(s)[(int64_t)by * nbc + bx] = (uint8_t)(e + 127);
    }
  };
  // Two register sets alternate (a loop body of two tiles), and so do the
  // two halves of red: a wave that still reads one half cannot be overtaken
  // by writes into it, which come two tiles (and a barrier) later.
  Raw8<InT> ra[4];
  uint32_t t = blockIdx.x;
  load_tile(t, ra);
  if constexpr (!PIPE) {
    process(t, ra, 0);
    return;
  }
  Raw8<InT> rb[4];
  const uint32_t step = gridDim.x;
  for (;;) {
    uint32_t tn = t + step;
    if (tn < ntiles) load_tile(tn, rb);
    process(t, ra, 0);
    if (tn >= ntiles) break;
    t = tn;
    tn = t + step;
    if (tn < ntiles) load_tile(tn, ra);
    process(t, rb, 1);
    if (tn >= ntiles) break;
    t = tn;
  }
}

// ---------------------------------------------------------------------------
// 32-element MX blocks along rows: 4 lanes x 8 elements per block, 16 blocks
// of one row per wavefront item.  RULE 1 = OCP floor exponent, whose scaled
// values may exceed fmax: those are counted (optional) and clamped before the
// cast, which is the saturation of the last bin.  RULE 0 = round-up exponent.
// ---------------------------------------------------------------------------
template <typename InT, int FMT, int RULE, bool COUNTS, int U>
__global__ __launch_bounds__(kThreads) void mx_kernel(
    const InT* __restrict__ x, int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
    uint8_t* __restrict__ s, uint8_t* __restrict__ cnt, uint32_t nblk, uint32_t ipr,
    uint32_t total_items) {
  constexpr float fmax = FmtInfo<FMT>::fmax;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t sub = lane & 3;
  const uint32_t slot = lane >> 2;
  // Known uniform: the item index math (row = item / items per row, addresses)
  // then runs on the scalar unit.
  const uint32_t wave = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t nwaves = gridDim.x * (kThreads / 64);
  for (uint32_t it = wave * U; it < total_items; it += nwaves * U) {
    float f[U][8];
    uint32_t row[U], blk[U];
    bool act[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t item = it + u;
      const uint32_t r = item / ipr;
      const uint32_t b = (item - r * ipr) * 16 + slot;
      row[u] = r;
      blk[u] = b;
      act[u] = item < total_items && b < nblk;
      if (act[u]) load8<false>(x + (int64_t)r * ldx + b * 32 + sub * 8, f[u]);
      else zero8(f[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = max(m, abs_bits(f[u][j]));
      m = max_quad(m);
      const int e = RULE == 1 ? scale_exp_floor<FMT>(m) : scale_exp_ceil<FMT>(m);
      const float sc = pow2_neg(e);
      float v[8];
      uint32_t n = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[j] = f[u][j] * sc;
        if (COUNTS) n += fabsf(v[j]) > fmax ? 1u : 0u;
        v[j] = __builtin_amdgcn_fmed3f(v[j], -fmax, fmax);
      }
      if (COUNTS) n = sum_quad(n);
      if (act[u]) {
        uint2 o;
        o.x = cvt4<FMT>(v[0], v[1], v[2], v[3]);
        o.y = cvt4<FMT>(v[4], v[5], v[6], v[7]);
        store_codes(q + (int64_t)row[u] * ldq + blk[u] * 32 + sub * 8, o);
        if (sub == 0) {
          s[(int64_t)row[u] * nblk + blk[u]] = (uint8_t)(e + 127);
          if (COUNTS) cnt[(int64_t)row[u] * nblk + blk[u]] = (uint8_t)n;
        }
      }
    }
  }
}

static uint32_t grid_for(uint64_t items, int per_wave) {
  const uint64_t waves = (items + per_wave - 1) / per_wave;
  uint64_t blocks = (waves + 3) / 4;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  return blocks ? (uint32_t)blocks : 1u;
}

}  // namespace quant_detail

using namespace quant_detail;

// ----------------------------------------------------------------- launchers

template <typename InT, int FMT, bool F32S>
static void row_dispatch(const void* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* q,
                         int64_t ldq, void* s, hipStream_t st) {
  constexpr int U = 2;
  const uint32_t ngroups = (uint32_t)((cols + 127) / 128);
  const uint32_t ipr = (ngroups + 3) / 4;
  const uint64_t items = (uint64_t)rows * ipr;
  const auto kern = stream_loads(rows, cols, sizeof(InT)) ? quant_row_kernel<InT, FMT, U, F32S, true>
                                                          : quant_row_kernel<InT, FMT, U, F32S, false>;
  hipLaunchKernelGGL(kern, dim3(grid_for(items, U)), dim3(kThreads), 0, st, (const InT*)x, (uint32_t)cols, ldx, q,
                     ldq, s, ngroups, ipr, (uint32_t)items);
}

template <bool F32S>
static void row_any(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                    int64_t ldq, void* s, hipStream_t st) {
  if (dtype == 1) {
    if (fmt == 0) row_dispatch<uint16_t, 0, F32S>(x, rows, cols, ldx, q, ldq, s, st);
    else row_dispatch<uint16_t, 1, F32S>(x, rows, cols, ldx, q, ldq, s, st);
  } else {
    if (fmt == 0) row_dispatch<float, 0, F32S>(x, rows, cols, ldx, q, ldq, s, st);
    else row_dispatch<float, 1, F32S>(x, rows, cols, ldx, q, ldq, s, st);
  }
}

void launch_quant_row(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                      uint8_t* q, int64_t ldq, uint8_t* s, hipStream_t st) {
  row_any<false>(x, dtype, rows, cols, ldx, fmt, q, ldq, s, st);
}

void launch_quant_row_f32s(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                           uint8_t* q, int64_t ldq, float* s, hipStream_t st) {
  row_any<true>(x, dtype, rows, cols, ldx, fmt, q, ldq, s, st);
}

template <typename InT, int FMT, bool F32S>
static void col_dispatch(const void* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* qt,
                         int64_t ldq, void* st, hipStream_t stream) {
  const uint32_t ngt = (uint32_t)((rows + 127) / 128);
  const dim3 grid((uint32_t)((cols + 127) / 128) * ngt);
  const auto kern = stream_loads(rows, cols, sizeof(InT)) ? quant_col_t_kernel<InT, FMT, F32S, true>
                                                          : quant_col_t_kernel<InT, FMT, F32S, false>;
  hipLaunchKernelGGL(kern, grid, dim3(kColThreads), 0, stream, (const InT*)x, (uint32_t)rows, (uint32_t)cols, ldx,
                     qt, ldq, st, ngt);
}

template <bool F32S>
static void col_any(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* qt,
                    int64_t ldq, void* st, hipStream_t stream) {
  if (dtype == 1) {
    if (fmt == 0) col_dispatch<uint16_t, 0, F32S>(x, rows, cols, ldx, qt, ldq, st, stream);
    else col_dispatch<uint16_t, 1, F32S>(x, rows, cols, ldx, qt, ldq, st, stream);
  } else {
    if (fmt == 0) col_dispatch<float, 0, F32S>(x, rows, cols, ldx, qt, ldq, st, stream);
    else col_dispatch<float, 1, F32S>(x, rows, cols, ldx, qt, ldq, st, stream);
  }
}

void launch_quant_col_t(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                        uint8_t* qt, int64_t ldq, uint8_t* st, hipStream_t stream) {
  col_any<false>(x, dtype, rows, cols, ldx, fmt, qt, ldq, st, stream);
}

void launch_quant_col_t_f32s(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                             uint8_t* qt, int64_t ldq, float* st, hipStream_t stream) {
  col_any<true>(x, dtype, rows, cols, ldx, fmt, qt, ldq, st, stream);
}

template <typename InT, int FMT>
static void dual_dispatch(const void* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* q, int64_t ldq,
                          uint8_t* s, uint8_t* qt, int64_t ldqt, uint8_t* st, hipStream_t stream) {
  const uint32_t ngc = (uint32_t)((cols + 127) / 128), ngt = (uint32_t)((rows + 127) / 128);
  const auto kern = stream_loads(rows, cols, sizeof(InT)) ? quant_dual_kernel<InT, FMT, true>
                                                          : quant_dual_kernel<InT, FMT, false>;
  hipLaunchKernelGGL(kern, dim3(ngc * ngt), dim3(kColThreads), 0, stream, (const InT*)x, (uint32_t)rows,
                     (uint32_t)cols, ldx, q, ldq, s, qt, ldqt, st, ngc, ngt);
}

void launch_quant_dual(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                       int64_t ldq, uint8_t* s, uint8_t* qt, int64_t ldqt, uint8_t* st, hipStream_t stream) {
  if (dtype == 1) {
    if (fmt == 0) dual_dispatch<uint16_t, 0>(x, rows, cols, ldx, q, ldq, s, qt, ldqt, st, stream);
    else dual_dispatch<uint16_t, 1>(x, rows, cols, ldx, q, ldq, s, qt, ldqt, st, stream);
  } else {
    if (fmt == 0) dual_dispatch<float, 0>(x, rows, cols, ldx, q, ldq, s, qt, ldqt, st, stream);
    else dual_dispatch<float, 1>(x, rows, cols, ldx, q, ldq, s, qt, ldqt, st, stream);
  }
}

template <typename InT, int FMT>
static void block_dual_dispatch(const void* w, int64_t rows, int64_t cols, int64_t ldw, uint8_t* q,
                                int64_t ldq, uint8_t* s, uint8_t* qt, int64_t ldqt, uint8_t* st,
                                hipStream_t stream) {
  const uint32_t nbc = (uint32_t)((cols + 127) / 128), nbr = (uint32_t)((rows + 127) / 128);
  const auto kern = stream_loads(rows, cols, sizeof(InT)) ? quant_block_dual_kernel<InT, FMT, true>
                                                          : quant_block_dual_kernel<InT, FMT, false>;
  hipLaunchKernelGGL(kern, dim3(nbc * nbr), dim3(kThreads), 0, stream, (const InT*)w, (uint32_t)rows,
                     (uint32_t)cols, ldw, q, ldq, s, qt, ldqt, st, nbc, nbr);
}

void launch_quant_block_dual(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw, int fmt,
                             uint8_t* q, int64_t ldq, uint8_t* s, uint8_t* qt, int64_t ldqt, uint8_t* st,
                             hipStream_t stream) {
  if (dtype == 1) {
    if (fmt == 0) block_dual_dispatch<uint16_t, 0>(w, rows, cols, ldw, q, ldq, s, qt, ldqt, st, stream);
    else block_dual_dispatch<uint16_t, 1>(w, rows, cols, ldw, q, ldq, s, qt, ldqt, st, stream);
  } else {
    if (fmt == 0) block_dual_dispatch<float, 0>(w, rows, cols, ldw, q, ldq, s, qt, ldqt, st, stream);
    else block_dual_dispatch<float, 1>(w, rows, cols, ldw, q, ldq, s, qt, ldqt, st, stream);
  }
}

template <typename InT, int FMT, bool F32S>
static void block_dispatch(const void* w, int64_t rows, int64_t cols, int64_t ldw, uint8_t* q,
                           int64_t ldq, void* s, hipStream_t stream) {
  const uint32_t nbc = (uint32_t)((cols + 127) / 128);
  const uint32_t ntiles = nbc * (uint32_t)((rows + 127) / 128);
  // Pipelined when the tiles outnumber the workgroups one round of the
  // one-tile form holds (four per CU): then tiles per workgroup as few as
  // let every workgroup be resident at once (three per CU with bf16 input,
  // two with fp32, whose prefetched tile takes twice the registers), spread
  // evenly.  (Fewer tiles, e.g. 840 for a 8960x1536 weight, ran 11 % slower
  // pipelined at two per workgroup.)
  const uint32_t cus = (uint32_t)device_cus();
  const bool pipe = !F32S && ntiles > 4 * cus;
  const uint32_t slots = (sizeof(InT) == 2 ? 3u : 2u) * cus;
  const uint32_t per = pipe ? (ntiles + slots - 1) / slots : 1;
  const dim3 grid((ntiles + per - 1) / per);
  const bool nt = stream_loads(rows, cols, sizeof(InT));
  const auto kern = pipe ? (nt ? quant_block_kernel<InT, FMT, F32S, true, !F32S>
                               : quant_block_kernel<InT, FMT, F32S, false, !F32S>)
                         : (nt ? quant_block_kernel<InT, FMT, F32S, true, false>
                               : quant_block_kernel<InT, FMT, F32S, false, false>);
  hipLaunchKernelGGL(kern, grid, dim3(kBlockThreads), 0, stream, (const InT*)w, (uint32_t)rows, (uint32_t)cols,
                     ldw, q, ldq, s, nbc, ntiles);
}

template <bool F32S>
static void block_any(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw, int fmt, uint8_t* q,
                      int64_t ldq, void* s, hipStream_t stream) {
  if (dtype == 1) {
    if (fmt == 0) block_dispatch<uint16_t, 0, F32S>(w, rows, cols, ldw, q, ldq, s, stream);
    else block_dispatch<uint16_t, 1, F32S>(w, rows, cols, ldw, q, ldq, s, stream);
  } else {
    if (fmt == 0) block_dispatch<float, 0, F32S>(w, rows, cols, ldw, q, ldq, s, stream);
    else block_dispatch<float, 1, F32S>(w, rows, cols, ldw, q, ldq, s, stream);
  }
}

void launch_quant_block(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw, int fmt,
                        uint8_t* q, int64_t ldq, uint8_t* s, hipStream_t stream) {
  block_any<false>(w, dtype, rows, cols, ldw, fmt, q, ldq, s, stream);
}

void launch_quant_block_f32s(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw, int fmt,
                             uint8_t* q, int64_t ldq, float* s, hipStream_t stream) {
  block_any<true>(w, dtype, rows, cols, ldw, fmt, q, ldq, s, stream);
}

template <typename InT, int FMT, int RULE, bool COUNTS>
static void mx_dispatch(const void* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* q, int64_t ldq,
                        uint8_t* s, uint8_t* counts, hipStream_t stream) {
  constexpr int U = 2;
  const uint32_t nblk = (uint32_t)(cols / 32);
  const uint32_t ipr = (nblk + 15) / 16;
  const uint64_t items = (uint64_t)rows * ipr;
  // Ordinary loads at every size: non-temporal ones made this kernel 15 %
  // slower on 64 MiB fp32 tensors.
  hipLaunchKernelGGL((mx_kernel<InT, FMT, RULE, COUNTS, U>), dim3(grid_for(items, U)), dim3(kThreads), 0,
                     stream, (const InT*)x, ldx, q, ldq, s, counts, nblk, ipr, (uint32_t)items);
}

template <typename InT, int FMT>
static void mx_dispatch_rule(const void* x, int64_t rows, int64_t cols, int64_t ldx, int rule, uint8_t* q,
                             int64_t ldq, uint8_t* s, uint8_t* counts, hipStream_t stream) {
  if (rule == 1) {
    if (counts) mx_dispatch<InT, FMT, 1, true>(x, rows, cols, ldx, q, ldq, s, counts, stream);
    else mx_dispatch<InT, FMT, 1, false>(x, rows, cols, ldx, q, ldq, s, counts, stream);
  } else {
    if (counts) mx_dispatch<InT, FMT, 0, true>(x, rows, cols, ldx, q, ldq, s, counts, stream);
    else mx_dispatch<InT, FMT, 0, false>(x, rows, cols, ldx, q, ldq, s, counts, stream);
  }
}

void launch_mx(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt, int rule,
               uint8_t* q, int64_t ldq, uint8_t* s, uint8_t* counts, hipStream_t stream) {
  if (dtype == 1) {
    if (fmt == 0) mx_dispatch_rule<uint16_t, 0>(x, rows, cols, ldx, rule, q, ldq, s, counts, stream);
    else mx_dispatch_rule<uint16_t, 1>(x, rows, cols, ldx, rule, q, ldq, s, counts, stream);
  } else {
    if (fmt == 0) mx_dispatch_rule<float, 0>(x, rows, cols, ldx, rule, q, ldq, s, counts, stream);
    else mx_dispatch_rule<float, 1>(x, rows, cols, ldx, rule, q, ldq, s, counts, stream);
  }
}

}  // namespace mxfp8
