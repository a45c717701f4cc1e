// gemm.hip -- block-scaled FP8 GEMM on CDNA4 MFMA (gfx950).
//
// C[m][n] = sum over 128-wide K blocks kb of
//           2^(sa(m,kb)-127) * 2^(sb(kb,n)-127) * sum_{k in kb} A[m][k] * B(k, n)
// with FP8 (E4M3 / E5M2) operands and fp32 accumulation: the FP8 GEMMs that
// consume per-token and per-block scaled operands ["A Comprehensive FP8
// Training Recipe for Reasoning-Enhanced Language Models", "What carries the
// argument"].
//
// Design (gfx950 specifics):
//  * One v_mfma_scale_f32_16x16x128_f8f6f4 covers exactly one 128-wide K
//    block.  Its E8M0 scale operands take the per-row A scale and the per-
//    column B scale of that block, so the per-block rescale happens inside the
//    matrix core and every K block accumulates straight into the fp32
//    accumulators (no separate partial-sum rescale).  The MFMA multiplies
//    products exactly and adds at most K/128 block results per output into
//    fp32, which keeps the error far below 2^-12 * sum|a*b|.
//  * Operands are swapped (B fragment first) so that each lane owns 4
//    consecutive output columns of one row: 16-byte (fp32) / 8-byte (bf16)
//    stores.
//  * Tiles move HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging),
//    double buffered: the loads for K block ks+1 are in flight while the
//    MFMAs of block ks run.  Rows of the [rows][128 B] LDS tiles are XOR-
//    swizzled in 16-byte chunks so that fragment reads (two ds_read_b128 per
//    lane) are bank-conflict free.
//  * B stored [K][N] (the dgrad case): the tile is kept as [128 k][BN bytes]
//    and read with ds_read_b64_tr_b8, which transposes 8x16-byte blocks across
//    a 16-lane group, giving each lane 8 consecutive k of one column.
//  * Workgroup ids are remapped so that each XCD (8 per device, own L2) walks
//    a contiguous band of tiles in grouped-row order.
#include "launch.hpp"

#include <stdint.h>

namespace mxfp8 {

namespace gemm_detail {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int kThreads = 256;  // 4 waves, arranged 2 x 2 over the tile

__device__ __forceinline__ uint32_t bf16_rne(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

// 16-byte chunk swizzle of the [rows][128 B] tiles: row r, logical chunk c
// lives at physical chunk c ^ ((r >> 1) & 7).  Sixteen consecutive rows read
// at one logical chunk then cover all 64 banks exactly once.
__device__ __forceinline__ uint32_t swz_rows(uint32_t r) { return (r >> 1) & 7; }

// Swizzle of the [128 k][BN bytes] tile for B stored [K][N]; CPR = BN / 16
// chunks per row.  The eight rows that one transposed read touches land on
// distinct chunks, and the two 16-lane halves of a wave use disjoint halves of
// the row when CPR == 16.
template <int CPR>
__device__ __forceinline__ uint32_t swz_kn(uint32_t k) {
  return CPR == 16 ? ((k & 7) | (((k >> 5) & 1) << 3)) : (k & 7);
}

// HBM -> LDS for one K block: each wave-instruction moves 1 KB (64 lanes x 16
// bytes) to consecutive LDS; the per-lane source addresses encode the swizzle.
template <int A_LOADS, int B_LOADS>
__device__ __forceinline__ void issue_tile_loads(uint8_t* smem, int a_bytes, int b_bytes, int wave,
                                                 const uint8_t* const (&a_src)[A_LOADS],
                                                 const uint8_t* const (&b_src)[B_LOADS], int ks, int64_t b_step,
                                                 int buf) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint8_t* a_dst = smem + buf * (a_bytes + b_bytes);
  uint8_t* b_dst = a_dst + a_bytes;
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j)
    __builtin_amdgcn_global_load_lds(a_src[j] + (int64_t)ks * 128, a_dst + (j * 4 + wave) * 1024, 16, 0, 0);
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j)
    __builtin_amdgcn_global_load_lds(b_src[j] + (int64_t)ks * b_step, b_dst + (j * 4 + wave) * 1024, 16, 0, 0);
#endif
}

// Scale bytes of K block ks for this lane's rows (A) and columns (B).
template <int MT, int NT>
__device__ __forceinline__ void load_scales(const uint8_t* const (&sa_src)[MT], const uint8_t* const (&sb_src)[NT],
                                            int64_t sb_step, int ks, int (&sa)[MT], int (&sb)[NT]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) sa[mt] = sa_src[mt][ks];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) sb[nt] = sb_src[nt][(int64_t)ks * sb_step];
}

template <int BM, int BN, int AFMT, int BFMT, bool BKN, bool BROW>
__global__ __launch_bounds__(kThreads) void gemm_bs_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ SA,
    const uint8_t* __restrict__ B, int64_t ldb, const uint8_t* __restrict__ SB, void* __restrict__ C,
    int64_t ldc, int out_bf16, int tiles_m, int tiles_n) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  constexpr int WM = BM / 2, WN = BN / 2;       // per-wave tile
  constexpr int MT = WM / 16, NT = WN / 16;     // 16x16 MFMA tiles per wave
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  constexpr int A_LOADS = A_BYTES / (kThreads * 16);
  constexpr int B_LOADS = B_BYTES / (kThreads * 16);
  constexpr int CPR = BN / 16;                  // 16-byte chunks per KN tile row
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * (A_BYTES + B_BYTES)];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile selection: XCD-contiguous bands, grouped rows within a band
  int wg = blockIdx.x;
  const int nwg = tiles_m * tiles_n;
  if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
  constexpr int GROUP = 8;
  const int group = wg / (GROUP * tiles_n);
  const int first = group * GROUP;
  const int gsz = min(tiles_m - first, GROUP);
  const int within = wg - group * GROUP * tiles_n;
  const int tm = first + within % gsz;
  const int tn = within / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int nkb = K >> 7;
  const int nnb = (N + 127) >> 7;

  // ---- per-lane global source addresses for the LDS loads (K block 0)
  const uint8_t* a_src[A_LOADS];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    const int row = (j * 4 + wave) * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ swz_rows(row);
    const int gm = min(m0 + row, M - 1);
    a_src[j] = A + (int64_t)gm * lda + lc * 16;
  }
  const uint8_t* b_src[B_LOADS];
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    if (!BKN) {
      const int row = (j * 4 + wave) * 8 + (lane >> 3);
      const int lc = (lane & 7) ^ swz_rows(row);
      const int gn = min(n0 + row, N - 1);
      b_src[j] = B + (int64_t)gn * ldb + lc * 16;
    } else {
      constexpr int RPI = 64 / CPR;  // k rows per wave-instruction
      const int krow = (j * 4 + wave) * RPI + lane / CPR;
      const int lc = (lane % CPR) ^ swz_kn<CPR>(krow);
      int col = n0 + lc * 16;
      if (col >= N) col = 0;
      b_src[j] = B + (int64_t)krow * ldb + col;
    }
  }
  const int64_t b_step = BKN ? (int64_t)128 * ldb : 128;

  // ---- scale sources
  const uint8_t* sa_src[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int gm = min(m0 + wm * WM + mt * 16 + (lane & 15), M - 1);
    sa_src[mt] = SA + (int64_t)gm * nkb;
  }
  const uint8_t* sb_src[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (BROW) {
      const int gn = min(n0 + wn * WN + nt * 16 + (lane & 15), N - 1);
      sb_src[nt] = SB + (int64_t)gn * nkb;
    } else {
      const int nb = min((n0 + wn * WN + nt * 16) >> 7, nnb - 1);
      sb_src[nt] = BKN ? SB + nb : SB + (int64_t)nb * nkb;
    }
  }
  const int64_t sb_step = (!BROW && BKN) ? nnb : 1;

  int sa_nxt[MT], sb_nxt[NT];

  v4f acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

  if (nkb > 0) {
    issue_tile_loads<A_LOADS, B_LOADS>(smem, A_BYTES, B_BYTES, wave, a_src, b_src, 0, b_step, 0);
    load_scales<MT, NT>(sa_src, sb_src, sb_step, 0, sa_nxt, sb_nxt);
  }

  const int g = lane >> 4;
  for (int ks = 0; ks < nkb; ++ks) {
    const int buf = ks & 1;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's LDS loads for block ks have landed
    __syncthreads();                // ... and every other wave's; buffer buf^1 is free
    int sa_cur[MT], sb_cur[NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sa_cur[mt] = sa_nxt[mt];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) sb_cur[nt] = sb_nxt[nt];

    const uint8_t* a_lds = smem + buf * (A_BYTES + B_BYTES);
    const uint8_t* b_lds = a_lds + A_BYTES;
    v8i af[MT], bfr[NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = wm * WM + mt * 16 + (lane & 15);
      const int sw = swz_rows(r);
      const v4i lo = *reinterpret_cast<const v4i*>(a_lds + r * 128 + (((2 * g) ^ sw) << 4));
      const v4i hi = *reinterpret_cast<const v4i*>(a_lds + r * 128 + (((2 * g + 1) ^ sw) << 4));
      af[mt] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (!BKN) {
        const int r = wn * WN + nt * 16 + (lane & 15);
        const int sw = swz_rows(r);
        const v4i lo = *reinterpret_cast<const v4i*>(b_lds + r * 128 + (((2 * g) ^ sw) << 4));
        const v4i hi = *reinterpret_cast<const v4i*>(b_lds + r * 128 + (((2 * g + 1) ^ sw) << 4));
        bfr[nt] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      } else {
        const int nsub = (wn * WN + nt * 16) >> 4;
        const int j = (lane & 15) >> 1, half = lane & 1;
        v2i part[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int k = 32 * g + 8 * t + j;
          const int off = k * BN + ((nsub ^ (int)swz_kn<CPR>(k)) << 4) + half * 8;
          part[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(b_lds + off));
        }
        bfr[nt] = v8i{part[0].x, part[0].y, part[1].x, part[1].y, part[2].x, part[2].y, part[3].x, part[3].y};
      }
    }

    if (ks + 1 < nkb) {
      issue_tile_loads<A_LOADS, B_LOADS>(smem, A_BYTES, B_BYTES, wave, a_src, b_src, ks + 1, b_step, buf ^ 1);
      load_scales<MT, NT>(sa_src, sb_src, sb_step, ks + 1, sa_nxt, sb_nxt);
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bfr[nt], af[mt], acc[mt][nt], BFMT, AFMT, 0, sb_cur[nt], 0, sa_cur[mt]);
  }

  // ---- epilogue: lane holds C[m][nb .. nb+3]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + wm * WM + mt * 16 + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int nb = n0 + wn * WN + nt * 16 + g * 4;
      const v4f v = acc[mt][nt];
      if (!out_bf16) {
        float* crow = reinterpret_cast<float*>(C) + (int64_t)m * ldc;
        if (nb + 3 < N) {
          *reinterpret_cast<v4f*>(crow + nb) = v;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (nb + i < N) crow[nb + i] = v[i];
        }
      } else {
        uint16_t* crow = reinterpret_cast<uint16_t*>(C) + (int64_t)m * ldc;
        if (nb + 3 < N) {
          uint2 o;
          o.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
          o.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
          *reinterpret_cast<uint2*>(crow + nb) = o;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (nb + i < N) crow[nb + i] = (uint16_t)bf16_rne(v[i]);
        }
      }
    }
  }
#endif
}

template <int BM, int BN, int AFMT, int BFMT, bool BKN, bool BROW>
void launch_tile(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa,
                 const uint8_t* b, int64_t ldb, const uint8_t* sb, void* c, int64_t ldc, int c_dtype,
                 hipStream_t stream) {
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bs_kernel<BM, BN, AFMT, BFMT, BKN, BROW>), dim3(tiles_m * tiles_n), dim3(kThreads),
                     0, stream, (int)M, (int)N, (int)K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype == 1 ? 1 : 0,
                     tiles_m, tiles_n);
}

template <int AFMT, int BFMT>
void launch_fmt(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa,
                const uint8_t* b, int64_t ldb, int b_layout, const uint8_t* sb, int b_scale_mode, void* c,
                int64_t ldc, int c_dtype, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  if (b_layout == 1)
    launch_tile<BM, BN, AFMT, BFMT, true, false>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype, stream);
  else if (b_scale_mode == 1)
    launch_tile<BM, BN, AFMT, BFMT, false, true>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype, stream);
  else
    launch_tile<BM, BN, AFMT, BFMT, false, false>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype, stream);
}

}  // namespace gemm_detail

using namespace gemm_detail;

void launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, int a_fmt,
                 const uint8_t* sa, const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
                 const uint8_t* sb, int b_scale_mode, void* c, int64_t ldc, int c_dtype,
                 hipStream_t stream) {
  if (a_fmt == 0 && b_fmt == 0)
    launch_fmt<0, 0>(M, N, K, a, lda, sa, b, ldb, b_layout, sb, b_scale_mode, c, ldc, c_dtype, stream);
  else if (a_fmt == 1 && b_fmt == 0)
    launch_fmt<1, 0>(M, N, K, a, lda, sa, b, ldb, b_layout, sb, b_scale_mode, c, ldc, c_dtype, stream);
  else if (a_fmt == 0 && b_fmt == 1)
    launch_fmt<0, 1>(M, N, K, a, lda, sa, b, ldb, b_layout, sb, b_scale_mode, c, ldc, c_dtype, stream);
  else
    launch_fmt<1, 1>(M, N, K, a, lda, sa, b, ldb, b_layout, sb, b_scale_mode, c, ldc, c_dtype, stream);
}

}  // namespace mxfp8
