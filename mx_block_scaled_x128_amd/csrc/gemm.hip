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
//  * v_mfma_scale_f32_32x32x64_f8f6f4 applies per-row E8M0 scales of both
//    operands inside the matrix core; two of them (two 64-wide K stages)
//    cover one 128-wide scale block with the same scale bytes.  Every block's
//    partial product therefore accumulates directly into the fp32
//    accumulators: no separate per-block rescale pass.  Products of FP8
//    values are exact; fp32 accumulation over 64-term MFMA sums keeps the
//    error far below 2^-12 * sum|a*b|.
//  * Operands are swapped (B fragment first), so each lane owns runs of 4
//    consecutive output columns of one row: 16-byte (fp32) / 8-byte (bf16)
//    stores.
//  * HBM -> LDS moves use global_load_lds_dwordx4 (no VGPR staging) into a
//    ring of STAGES buffers, STAGES stages ahead of the MFMAs.  Fragments are
//    double-buffered in registers: the next stage's ds_reads are interleaved
//    into the current stage's MFMA stream.  One barrier per 64-wide stage.
//  * Rows of the [rows][64 B] LDS tiles are XOR-swizzled in 16-byte chunks so
//    fragment reads (two ds_read_b128 per lane) are bank-conflict free.
//  * B stored [K][N] (the data-gradient case): the stage tile is kept as
//    [64 k][BN bytes] and read with ds_read_b64_tr_b8, which transposes an
//    8 x 16-byte block across a 16-lane group and hands each lane 8
//    consecutive k of one column.
//  * Workgroup ids are remapped so each XCD (8 per device, own L2) walks a
//    contiguous band of tiles in grouped-row order.
//  * Source addresses are a wave-uniform (SGPR) tile base plus 32-bit per-lane
//    offsets, so the address registers do not compete with the fragments.
#include "launch.hpp"

#include <stdint.h>


// One translation unit can hold every kernel (MXFP8_GEMM_FMT undefined), or
// the build compiles this file once per (A format, B format) pair,
// MXFP8_GEMM_FMT = 2 * a_fmt + b_fmt, in parallel, plus once with
// MXFP8_GEMM_FMT = -1 for the host dispatch alone.
#ifndef MXFP8_GEMM_FMT
#define MXFP8_GEMM_FMT 4
#endif

namespace mxfp8 {

namespace gemm_detail {

template <int AFMT, int BFMT>
void launch_fmt(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa,
                const uint8_t* b, int64_t ldb, int b_layout, const uint8_t* sb, int b_scale_mode, void* c,
                int64_t ldc, int c_dtype, hipStream_t stream);
template <int AFMT, int BFMT>
void launch_f32s_fmt(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa,
                     const uint8_t* b, int64_t ldb, int b_layout, const uint8_t* sb, int b_scale_mode, void* c,
                     int64_t ldc, int c_dtype, hipStream_t stream);
template <int AFMT, int BFMT>
void launch_mx_fmt(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa,
                   const uint8_t* b, int64_t ldb, const uint8_t* sb, void* c, int64_t ldc, int c_dtype,
                   hipStream_t stream);

#if MXFP8_GEMM_FMT >= 0

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int kThreads = 256;  // 4 waves, arranged 2 x 2 over the tile

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest-even bf16, packed (lo in bits 0-15):
// one v_cvt_pk_bf16_f32 (the default round mode is nearest-even; fp32
// subnormals are kept, and bf16 has fp32's exponent range).
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2bf));
}

// [rows][128 B] K-block tiles: row r, logical 16-byte chunk c at physical
// chunk c ^ ((r >> 1) & 7); sixteen consecutive rows read at one logical
// chunk hit 16 distinct 16-byte bank groups (two rows span all 64 banks).
__device__ __forceinline__ int swz128(int r) { return (r >> 1) & 7; }

// [64 k][BN bytes] stage tiles of B stored [K][N] (CPR = BN / 16 chunks per
// row): chunk c of row k at physical chunk c ^ s(k), s(k) even, so the two
// 16-column halves of a 32-column fragment (chunks 2p, 2p+1) and the eight
// rows of one transposed read cover 16 distinct bank groups.
template <int CPR>
__device__ __forceinline__ int swz_kn(int k) {
  return CPR == 16 ? 2 * (k & 7) : 2 * ((k >> 1) & 3);
}

// Retire this wave's VMEM loads older than the N most recent ones and all of
// its LDS reads, then meet every other wave.  The wait is the compiler-visible
// builtin (keeps the compiler's counter bookkeeping exact); the barrier is a
// bare s_barrier with a memory clobber, since __syncthreads()'s release fence
// would also drain every in-flight stage of LDS-bound loads.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(N >= 0 && N <= 63, "vmcnt");
  __builtin_amdgcn_sched_barrier(0);  // nothing (MFMAs included) crosses the stage boundary
  // gfx9 s_waitcnt: vmcnt[3:0] + vmcnt[5:4] at [15:14], expcnt[6:4] = 7 (none), lgkmcnt[11:8] = 0
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// Hides a value from the optimiser.  LDS read addresses are written as
// ring_slot + opaque lane offset + constant, so every read stays a short
// address expression on one named ring array: the backend then knows which
// slot each read touches and waits only for the loads into that slot.  (A
// long chain of partial sums shared between slots loses that knowledge and
// each read would drain every LDS-bound load in flight.)
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
  return x;
}

// Same for a wave-uniform pointer, kept in scalar registers.  HBM sources
// are written as (this per-stage uniform base) + 32-bit lane offset, which
// selects the scalar-base + vector-offset load form; otherwise loop-invariant
// code motion re-associates them into one 64-bit vector address per load,
// which costs two VGPRs each for the life of the loop.
__device__ __forceinline__ const uint8_t* uniform_opaque(const uint8_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+s"(p));
#endif
  return p;
}

// Lets the last MFMA retire before anything reads its accumulators.  The
// compiler's wait between a 32x32x64 scaled MFMA and a read of its result is
// too short for the last result registers: without this pad the epilogue
// stored acc[..][15] of the final MFMA without the last stage's contribution
// (two output columns per tile, reproducibly).  64 wait states cover the
// whole 16-pass operation.  Called at the end of every path out of the K
// loop, so that the accumulator copies the compiler places where the paths
// merge come after it.
__device__ __forceinline__ void mfma_retire_pad() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// Fraction (in quarters) of a stage's MFMAs over which the next stage's
// fragment reads are spread.
#ifndef MXFP8_GEMM_DS_SPAN
#define MXFP8_GEMM_DS_SPAN 3
#endif
// Fraction (in quarters) of the second stage's MFMAs over which the loads of
// the K block two ahead are spread (earlier loads have longer to land before
// the next K block's wait).
#ifndef MXFP8_GEMM_DMA_SPAN
#define MXFP8_GEMM_DMA_SPAN 4
#endif

// LDS of one tile body (bytes): two K-block buffers of PB bytes each, and the
// scale-group areas (SGRP bytes).  See gemm_tile for the layouts.
template <int BM, int BN>
struct TileLds {
  static constexpr int A_ST = BM * 128, B_ST = BN * 128;
  static constexpr int STG = 4 * 32 * (BN / 2 * 4);  // epilogue staging (fp32 strips)
  static constexpr int PB = A_ST + B_ST > STG ? A_ST + B_ST : STG;
  static constexpr int SGRP = 2 * 2 * kThreads * 4 * 4;
};

// MXS: MX operands -- scales per (row, 32-wide K block) for A ([M][K/32])
// and for B stored [N][K] ([N][K/32]); otherwise one scale per 128-wide K
// block (A [M][K/128]; B per row or per 128x128 tile of its storage).
// F32S: those 128-wide block scales are fp32 values, not powers of two (the
// "FP8 with an FP32 scale" variant): each K block's product runs through the
// matrix cores with unit scales into a temporary tile, which is then added
// into the accumulators times the block's scale product (one FMA per
// element, with a per-column multiply when B's scales are per column).
//
// gemm_tile is the body of one workgroup's tile (work item wg of nwg in its
// launch); the kernels below host it on their own LDS arrays (kbuf0, kbuf1:
// TileLds::PB bytes each, sgrp: TileLds::SGRP bytes, all 1024-byte aligned),
// one array per buffer so that every access names its buffer.
template <int BM, int BN, int STAGES, int AFMT, int BFMT, bool BKN, bool BROW, bool MXS, bool F32S, bool WS>
__device__ __forceinline__ void gemm_tile(
    int M, int N, int K, const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ SA,
    const uint8_t* __restrict__ B, int64_t ldb, const uint8_t* __restrict__ SB, void* __restrict__ C,
    int64_t ldc, int out_bf16, int tiles_m, int tiles_n, int tile_first, int sm, int sn, int wg_in, int nwg_in,
    uint8_t* kbuf0, uint8_t* kbuf1, uint8_t* sgrp) {
#if defined(__HIP_DEVICE_COMPILE__)  // device code only
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MT = WM / 32, NT = WN / 32;          // 32x32 MFMA tiles per wave
  static_assert(!MXS || (!BKN && BROW), "MX scales: B stored [N][K], scales per row");
  static_assert(!F32S || (BM == 128 && BN == 128 && !MXS), "fp32 scales: 128x128 tiles");
  // Scale values per B fragment held by a lane: one, except for fp32
  // per-column scales, where a lane's 16 accumulator columns each have one.
  constexpr int SBP = (F32S && BROW) ? 16 : 1;
  // LDS: two K-block buffers, each holding both 64-wide stages of one
  // 128-wide K block: the A tile [BM][128 B] and the B tile ([BN][128 B], or
  // [128 k][BN B] when B is [K][N]).  Whole 128-byte rows per load
  // instruction: HBM/L2 lines are 128 bytes, and loading a row's two 64-byte
  // halves in different stages fetched every line twice.  (A buffer also
  // hosts the epilogue's staging, hence its size.)
  constexpr int KBB = 128;                           // K bytes per buffer row
  constexpr int A_ST = TileLds<BM, BN>::A_ST, B_ST = TileLds<BM, BN>::B_ST;
  constexpr int PB = TileLds<BM, BN>::PB;
  constexpr int A_LOADS = A_ST / (kThreads * 16), B_LOADS = B_ST / (kThreads * 16);  // per K block, per thread
  constexpr int CPR = BN / 16;
  static_assert(BM % 64 == 0 && BN % 64 == 0 && A_LOADS >= 1 && B_LOADS >= 1, "tile");
  static_assert(BM <= kThreads && BN <= kThreads, "one scale entity per lane quarter");
  static_assert(A_LOADS + B_LOADS + 8 <= 63, "vmcnt range");
  // Scale groups: the scales of 4 consecutive K blocks for each of 256 tile
  // rows (A) and columns (B), double-buffered.  Loading 4 K blocks at a time
  // touches each row's scale line once per 4 K blocks instead of once per K
  // block (rows are nkb bytes apart in [rows][K/128] scales).  A 1-byte
  // LDS-bound load writes each lane's byte zero-extended into its own dword;
  // a 4-byte one writes the lane's 4 bytes.  An operand's group area holds
  // one of three layouts:
  //  * rows: scales per row of the operand's [rows][K] storage (A; B with
  //    per-row or MX scales).  Entity e's K block 4g + s in the dword at
  //    16 e + 4 s (MXS: that K block's four 32-wide block scales).  Loads:
  //    instruction q = 4 wave + j covers e = 16 q + lane / 4, s = lane % 4.
  //  * wide rows (WS: one E8M0 byte per K block, K blocks a multiple of 4,
  //    scale arrays 4-byte aligned): entity e's four bytes (s = 0..3) in the
  //    dword at 4 e, one 4-byte load per lane (entity 64 wave + lane), one
  //    instruction per operand and wave instead of four, and the 32 rows of
  //    a fragment read 32 consecutive dwords (no bank conflicts; the rows
  //    layout's 16-byte stride costs ~10 conflict cycles per read).
  //  * blocks: B scales per 128 x 128 block of its storage.  A tile's columns
  //    span at most two scale blocks, n0 / 128 + c (c = 0, 1), and each wave's
  //    columns lie in one of them, c = wn * WN / 128.  Each wave loads the
  //    group's 8 values into its own 256-byte row, (K block s, block c) in
  //    dword 2 s + c (lanes 8..63 repeat lanes 0..7), and reads its value with
  //    one same-address (broadcast) read per K block.  One instruction per
  //    wave instead of four.
  constexpr bool B_ROWS = BROW || MXS;
  static_assert(!WS || (!MXS && !F32S), "wide scale loads: one E8M0 byte per K block");
  constexpr int SG_OP = kThreads * 4 * 4;            // one operand's group area (bytes)
  constexpr int SG = 2 * SG_OP;                      // A then B
  static_assert(2 * SG == TileLds<BM, BN>::SGRP, "scale group areas");
  (void)STAGES;

  // Every access names its buffer with a compile-time constant (the loops
  // below are unrolled so that it does), so the compiler can tell the buffers
  // apart and does not drain in-flight LDS-bound loads into one buffer before
  // reading the other.
  auto buf_ptr = [&](int p) __attribute__((always_inline)) -> uint8_t* { return p == 0 ? kbuf0 : kbuf1; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // known uniform: LDS destinations stay scalar
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile of this workgroup.  Tiles are enumerated over a grid of
  // tiles_m x tiles_n cells of (BM << sm) x (BN << sn), in groups of GROUP
  // cell rows walked column by column; this launch covers cells tile_first,
  // tile_first + 1, ... and each cell as 2^sm x 2^sn BM x BN sub-tiles (one
  // workgroup each; sm = sn = 0: the cell itself).  Workgroup ids are first
  // remapped so that each XCD (ids are dealt round-robin to the 8 XCDs)
  // walks a contiguous band of that order.
  int wg = wg_in;
  const int nwg = nwg_in;
  if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
  const int cell = tile_first + (wg >> (sm + sn));
  const int sub = wg & ((1 << (sm + sn)) - 1);
  constexpr int GROUP = 4;  // measured against 2, 8 and 16: 4 is 0-2 % faster than 8, the others slower
  const int group = cell / (GROUP * tiles_n);
  const int first = group * GROUP;
  const int gsz = min(tiles_m - first, GROUP);
  const int within = cell - group * GROUP * tiles_n;
  const int m0 = (((first + within % gsz) << sm) + (sub >> sn)) * BM;
  const int n0 = (((within / gsz) << sn) + (sub & ((1 << sn) - 1))) * BN;
  if (m0 >= M || n0 >= N) return;  // a sub-tile past the matrix edge (uniform per workgroup)

  const int nkb = K >> 7;   // 128-wide K blocks (= scale blocks)
  const int nnb = (N + 127) >> 7;

  // ---- HBM -> LDS sources: uniform tile bases + per-lane 32-bit offsets.
  // Each wave-instruction fills 1 KB of LDS in lane order: 8 rows of 128
  // bytes (lane l: row l >> 3, physical chunk l & 7, which holds logical
  // chunk (l & 7) ^ swz128(row)).  Rows past M / N are clamped (their results
  // are dropped).
  const uint8_t* a_base = A + (int64_t)m0 * lda;
  uint32_t a_off[A_LOADS];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    const int row = (j * 4 + wave) * 8 + (lane >> 3);
    const int lc = (lane & 7) ^ swz128(row);
    a_off[j] = (uint32_t)((min(m0 + row, M - 1) - m0) * lda + lc * 16);
  }
  const uint8_t* b_base = BKN ? B : B + (int64_t)n0 * ldb;
  uint32_t b_off[B_LOADS];
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    if (!BKN) {
      const int row = (j * 4 + wave) * 8 + (lane >> 3);
      const int lc = (lane & 7) ^ swz128(row);
      b_off[j] = (uint32_t)((min(n0 + row, N - 1) - n0) * ldb + lc * 16);
    } else {
      constexpr int RPI = 64 / CPR;  // k rows per wave-instruction
      const int krow = (j * 4 + wave) * RPI + lane / CPR;
      const int lc = (lane % CPR) ^ swz_kn<CPR>(krow);
      int col = n0 + lc * 16;
      if (col >= N) col = 0;
      b_off[j] = (uint32_t)(krow * ldb + col);
    }
  }
  const int64_t b_step = BKN ? (int64_t)KBB * ldb : KBB;

  // Scale sources of group grp (layouts above).  K blocks past the last one
  // and rows past M / N are clamped to the last ones.
  const int srow = (MXS || F32S) ? 4 * nkb : nkb;  // scale bytes per row of A (and of per-row B scales)
  const uint8_t* sa_base = uniform_opaque(SA + (int64_t)m0 * srow);
  const uint8_t* sb_base = uniform_opaque(BROW ? SB + (int64_t)n0 * srow : SB);
  auto sdma_group = [&](int grp) __attribute__((always_inline)) {
    uint8_t* area = sgrp + (grp & 1) * SG;
    if constexpr (WS) {
      const int e = wave * 64 + lane;
      const int kb4 = 4 * min(grp, (nkb >> 2) - 1);
      __builtin_amdgcn_global_load_lds(sa_base + (uint32_t)(min(e, M - 1 - m0) * nkb + kb4), area + wave * 256, 4,
                                       0, 0);
      if constexpr (BROW)
        __builtin_amdgcn_global_load_lds(sb_base + (uint32_t)(min(e, N - 1 - n0) * nkb + kb4),
                                         area + SG_OP + wave * 256, 4, 0, 0);
    } else {
      const int kbs = min(4 * grp + (lane & 3), nkb - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = (wave * 4 + j) * 16 + (lane >> 2);
        if (MXS || F32S) {
          const uint32_t off = (uint32_t)(min(e, M - 1 - m0) * srow + 4 * kbs);
          __builtin_amdgcn_global_load_lds(sa_base + off, area + (wave * 4 + j) * 256, 4, 0, 0);
        } else {
          const uint32_t off = (uint32_t)(min(e, M - 1 - m0) * nkb + kbs);
          __builtin_amdgcn_global_load_lds(sa_base + off, area + (wave * 4 + j) * 256, 1, 0, 0);
        }
      }
      if constexpr (B_ROWS) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = (wave * 4 + j) * 16 + (lane >> 2);
          if constexpr (MXS || F32S) {
            const uint32_t off = (uint32_t)(min(e, N - 1 - n0) * srow + 4 * kbs);
            __builtin_amdgcn_global_load_lds(sb_base + off, area + SG_OP + (wave * 4 + j) * 256, 4, 0, 0);
          } else {
            const uint32_t off = (uint32_t)(min(e, N - 1 - n0) * nkb + kbs);
            __builtin_amdgcn_global_load_lds(sb_base + off, area + SG_OP + (wave * 4 + j) * 256, 1, 0, 0);
          }
        }
      }
    }
    if constexpr (!B_ROWS) {
      const int kbs = min(4 * grp + ((lane & 7) >> 1), nkb - 1);
      const int nb = min((n0 >> 7) + (lane & 1), nnb - 1);
      const uint32_t idx = (uint32_t)(BKN ? kbs * nnb + nb : nb * nkb + kbs);
      if constexpr (F32S)
        __builtin_amdgcn_global_load_lds(sb_base + 4 * idx, area + SG_OP + wave * 256, 4, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(sb_base + idx, area + SG_OP + wave * 256, 1, 0, 0);
    }
  };

  // LDS-bound loads of K block kb into buffer p, one instruction per item:
  // A_LOADS loads of A, then B_LOADS of B.
  constexpr int DMA_ITEMS = A_LOADS + B_LOADS;
  struct Src {
    const uint8_t *a, *b;
  };
  auto dma_src = [&](int kb) __attribute__((always_inline)) {
    Src src;
    src.a = uniform_opaque(a_base + (int64_t)kb * KBB);
    src.b = uniform_opaque(b_base + (int64_t)kb * b_step);
    return src;
  };
  // The lane offsets are redefined (opaquely, in place) at each use: kept
  // loop-invariant, they were widened to 64 bits outside the K loop (two
  // VGPRs each, plus a 64-bit add per load) instead of feeding the
  // scalar-base + 32-bit-offset form of the load.
  auto dma_item = [&](int p, const Src& src, int item) __attribute__((always_inline)) {
    uint8_t* buf = buf_ptr(p);
    if (item < A_LOADS) {
      a_off[item] = opaque(a_off[item]);
      __builtin_amdgcn_global_load_lds(src.a + a_off[item], buf + (item * 4 + wave) * 1024, 16, 0, 0);
    } else {
      const int j = item - A_LOADS;
      b_off[j] = opaque(b_off[j]);
      __builtin_amdgcn_global_load_lds(src.b + b_off[j], buf + A_ST + (j * 4 + wave) * 1024, 16, 0, 0);
    }
  };
  auto dma_kblock = [&](int p, int kb) __attribute__((always_inline)) {
    const Src src = dma_src(kb);
#pragma unroll
    for (int item = 0; item < DMA_ITEMS; ++item) dma_item(p, src, item);
  };

  // Scale operands of K block kb (from its group's area).  With MXS, lane
  // half g reads the 32-wide block scales 2g and 2g+1 of the K block (the
  // chunks whose scale it supplies in the block's two stages, see below);
  // stage h selects byte h with the MFMA's operand select.  Fragment mt's
  // rows are entities wm * WM + 32 mt + lane % 32 (likewise for B columns).
  const int g = lane >> 5;
  constexpr int ROW_E = WS ? 4 : 16;                 // bytes per entity in a rows layout
  const uint32_t sa_rd = opaque(ROW_E * (wm * WM + (lane & 31)) + (MXS ? 2 * g : 0));
  const uint32_t sb_rd = opaque(SG_OP + (B_ROWS ? ROW_E * (wn * WN + (lane & 31)) + (MXS ? 2 * g : 0)
                                                : wave * 256 + 4 * ((wn * WN) >> 7)));
  // With F32S and per-column B scales, lane half g reads the scales of its
  // 16 accumulator columns 8q + 4g + j (q, j = 0..3) of each fragment.
  const uint32_t sbc_rd = opaque(SG_OP + 16 * (wn * WN + 4 * g));
  auto read_scale = [&](const uint8_t* p, bool byte) __attribute__((always_inline)) -> int {
    if (byte) return (int)*p;
    if (MXS) return (int)*reinterpret_cast<const uint16_t*>(p);
    return *reinterpret_cast<const int*>(p);
  };
  auto read_scales = [&](int kb, int (&sa)[MT], int (&sb)[NT * SBP]) __attribute__((always_inline)) {
    const uint8_t* area = sgrp + ((kb >> 2) & 1) * SG;
    const int ks = kb & 3;
    const uint8_t* ar = area + (WS ? ks : 4 * ks);
    const uint8_t* br = area + (B_ROWS ? (WS ? ks : 4 * ks) : 8 * ks);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sa[mt] = read_scale(ar + sa_rd + mt * 32 * ROW_E, WS);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if constexpr (SBP == 16) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sb[nt * 16 + r] = *reinterpret_cast<const int*>(br + sbc_rd + 16 * (nt * 32 + 8 * (r >> 2) + (r & 3)));
      } else if constexpr (B_ROWS) {
        sb[nt] = read_scale(br + sb_rd + nt * 32 * ROW_E, WS);
      } else {
        sb[nt] = nt == 0 ? *reinterpret_cast<const int*>(br + sb_rd) : sb[0];  // one block per wave
      }
    }
  };

  v16f acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.0f;
  // F32S: each K block's unscaled product, per fragment pair.
  constexpr int TM = F32S ? MT : 1, TN = F32S ? NT : 1;
  v16f tmp[TM][TN];
#pragma unroll
  for (int mt = 0; mt < TM; ++mt)
#pragma unroll
    for (int nt = 0; nt < TN; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmp[mt][nt][i] = 0.0f;
  // F32S: acc[mt][nt] += tmp[mt][nt] * (block scale of the row x that of
  // each column).  Lane l's 16 accumulators of a fragment pair are row l & 31
  // and columns 8q + 4(l >> 5) + j of the 32x32 block (register 4q + j).
  auto apply = [&](int mt, int nt, const int (&ps_a)[MT], const int (&ps_b)[NT * SBP])
                   __attribute__((always_inline)) {
    if constexpr (F32S) {
      const float fa = __int_as_float(ps_a[mt]);
      if constexpr (SBP == 16) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[mt][nt][r] = __builtin_fmaf(tmp[mt][nt][r], fa * __int_as_float(ps_b[nt * 16 + r]), acc[mt][nt][r]);
      } else {
        const float f = fa * __int_as_float(ps_b[nt]);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][nt][r] = __builtin_fmaf(tmp[mt][nt][r], f, acc[mt][nt][r]);
      }
    }
  };

  // Fragments of one 64-wide stage (half h of a K block).  Lane l holds, for
  // its row (A) / column (B) l & 31, 32 K bytes as two 16-byte parts (its
  // first and last four registers), for both operands (the pairing the MFMA
  // needs).  The matrix core's own K order: lane half g = l >> 5 holds k
  // 16 g .. +15 in part 0 and 32 + 16 g .. +15 in part 1, and with scales per
  // 32 k the first 32 (part 0 of both halves) take the scale of lanes 0-31,
  // the last 32 that of lanes 32-63 (measured: a product placed in part 1 of
  // half 0 is scaled by the upper lanes' byte).  With MXS, stage h puts the
  // K block's 32-wide chunk h in part 0 and chunk 2 + h in part 1, so lane
  // half g's scales over the two stages are chunks 2g and 2g + 1: adjacent
  // bytes, one 16-bit read.  Without MXS (one scale per 128-wide block) any
  // K order shared by A and B gives the same sums; stage h then takes bytes
  // 64 h .. +63.  One LDS read
  // per item: A items 2*mt + part (16 bytes each), then B items (two 16-byte
  // parts per fragment, or four 8-byte transposed parts when B is [K][N]).
  constexpr int B_PARTS = BKN ? 4 : 2;
  constexpr int DS_ITEMS = 2 * MT + B_PARTS * NT;
  // Per-lane read offsets within a buffer, per stage half (the 32-row /
  // 32-column step of a fragment and the 8-row step of a transposed part are
  // added as constants: neither changes the swizzle, which depends only on
  // low row bits).
  uint32_t a_rd[2][2], b_rd[2][BKN ? NT : 2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const int r = wm * WM + (lane & 31);
      const int unit = MXS ? 4 * part + 2 * h + g : 4 * h + 2 * g + part;  // 16-byte unit of the row
      a_rd[h][part] = opaque(r * KBB + ((unit ^ swz128(r)) << 4));
    }
  if (!BKN) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        const int r = wn * WN + (lane & 31);
        const int unit = MXS ? 4 * part + 2 * h + g : 4 * h + 2 * g + part;
        b_rd[h][part] = opaque(A_ST + r * KBB + ((unit ^ swz128(r)) << 4));
      }
  } else {
    // 16-lane group grp covers columns 16*(grp&1) .. +15 and k half grp>>1;
    // lane pair (2j, 2j+1) points at row k of that block, bytes 0-7 / 8-15.
    const int grp = lane >> 4, j = (lane & 15) >> 1, half = lane & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 64 * h + 32 * (grp >> 1) + j;
#pragma unroll
      for (int nt = 0; nt < (BKN ? NT : 0); ++nt) {
        const int nsub = ((wn * WN + nt * 32) >> 4) + (grp & 1);
        b_rd[h][nt] = opaque(A_ST + k * BN + ((nsub ^ swz_kn<CPR>(k)) << 4) + half * 8);
      }
    }
  }
  auto ds_item = [&](int p, int h, int item, v8i (&af)[MT], v8i (&bfr)[NT]) __attribute__((always_inline)) {
    const uint8_t* buf = buf_ptr(p);
    if (item < 2 * MT) {
      const int mt = item >> 1, part = item & 1;
      const v4i v = *reinterpret_cast<const v4i*>(buf + a_rd[h][part] + mt * 32 * KBB);
      if (part == 0) af[mt].s0123 = v;
      else af[mt].s4567 = v;
    } else if (!BKN) {
      const int nt = (item - 2 * MT) >> 1, part = item & 1;
      const v4i v = *reinterpret_cast<const v4i*>(buf + b_rd[h][part] + nt * 32 * KBB);
      if (part == 0) bfr[nt].s0123 = v;
      else bfr[nt].s4567 = v;
    } else {
      // part t: k rows 8t .. 8t+7 of the lane's k half
      const int nt = (item - 2 * MT) >> 2, t = (item - 2 * MT) & 3;
      const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(buf + b_rd[h][nt] + 8 * t * BN));
      if (t == 0) bfr[nt].s01 = v;
      else if (t == 1) bfr[nt].s23 = v;
      else if (t == 2) bfr[nt].s45 = v;
      else bfr[nt].s67 = v;
    }
  };
  auto read_frags = [&](int p, int h, v8i (&af)[MT], v8i (&bfr)[NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int item = 0; item < DS_ITEMS; ++item) ds_item(p, h, item, af, bfr);
  };

  // One stage as an explicit instruction stream: MFMA i, then the LDS reads
  // and HBM->LDS loads whose turn comes after it.  The loads are spread
  // evenly over the whole stage and the next stage's fragment reads over its
  // first DS_SPAN MFMAs: an LDS-bound load stalls this wave's in-order issue
  // whenever the CU's load path is busy, and a burst of them starves the
  // MFMA pipe.  sched_barrier(0) keeps the order.
  constexpr int MFMAS = MT * NT;
  constexpr int DS_SPAN = MFMAS * MXFP8_GEMM_DS_SPAN / 4 > 0 ? MFMAS * MXFP8_GEMM_DS_SPAN / 4 : 1;
  constexpr int DMA_SPAN = MFMAS * MXFP8_GEMM_DMA_SPAN / 4 > 0 ? MFMAS * MXFP8_GEMM_DMA_SPAN / 4 : 1;
  // The stage multiplies fragments (ca, cb) with scales (csa, csb).
  // dma_p >= 0: load K block dma_kb into buffer dma_p meanwhile.
  // rd_p >= 0: read the fragments of stage half rd_h of buffer rd_p into
  // (na, nb); with do_sc also K block sc_kb's scales into (nsa, nsb).
  // grp >= 0: load scale group grp.
  // F32S: the first stage of a K block first adds the previous K block's
  // temporaries into the accumulators (with that block's scales, still in
  // (nsa, nsb) until this block's second stage reads the next ones), one
  // fragment pair before each MFMA that overwrites its temporary; at least
  // three MFMAs separate each temporary's last write from that read.
  auto stage = [&](int cur_h, int dma_p, int dma_kb, int rd_p, int rd_h, bool do_sc, int sc_kb, int grp,
                   const v8i (&ca)[MT],
                   const v8i (&cb)[NT], v8i (&na)[MT], v8i (&nb)[NT], const int (&csa)[MT],
                   const int (&csb)[NT * SBP], int (&nsa)[MT], int (&nsb)[NT * SBP]) __attribute__((always_inline)) {
    Src src = {nullptr, nullptr};
    if (dma_p >= 0) src = dma_src(dma_kb);
#pragma unroll
    for (int i = 0; i < MFMAS; ++i) {
      const int mt = i / NT, nt = i % NT;
      if constexpr (F32S) {
        if (cur_h == 0) {
          apply(mt, nt, nsa, nsb);
          tmp[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cb[nt], ca[mt], v16f{}, BFMT, AFMT, 0,
                                                                       127, 0, 127);
        } else {
          tmp[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cb[nt], ca[mt], tmp[mt][nt], BFMT, AFMT,
                                                                       0, 127, 0, 127);
        }
      } else if (MXS && cur_h == 1) {
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cb[nt], ca[mt], acc[mt][nt], BFMT, AFMT, 1,
                                                                     csb[nt], 1, csa[mt]);
      } else {
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cb[nt], ca[mt], acc[mt][nt], BFMT, AFMT, 0,
                                                                     csb[nt], 0, csa[mt]);
      }
      if (rd_p >= 0 && do_sc && i == 0) read_scales(sc_kb, nsa, nsb);
      if (grp >= 0 && i == 0) sdma_group(grp);  // after the scale read: same array
#pragma unroll
      for (int item = 0; item < DS_ITEMS; ++item)
        if (rd_p >= 0 && item * DS_SPAN / DS_ITEMS == i) ds_item(rd_p, rd_h, item, na, nb);
#pragma unroll
      for (int item = 0; item < DMA_ITEMS; ++item)
        if (dma_p >= 0 && item * DMA_SPAN / DMA_ITEMS == i) dma_item(dma_p, src, item);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Two register sets each for fragments (stage parity) and scales (K block
  // parity); the code below alternates them, so nothing is copied.
  v8i fa0[MT], fb0[NT], fa1[MT], fb1[NT];
  int sa0[MT], sb0[NT * SBP], sa1[MT], sb1[NT * SBP];
  if constexpr (F32S) {  // the "previous K block" of the first one: zero temporaries, zero scales
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sa1[mt] = 0;
#pragma unroll
    for (int i = 0; i < NT * SBP; ++i) sb1[i] = 0;
  }

  // ---- schedule.  Each K block's first stage
  // multiplies while the second stage's fragments are read.  At the top of
  // its second stage every wave waits for all its loads (K block kb+1,
  // issued one K block earlier) and meets the others: K block kb+1 has then
  // landed everywhere, and nobody reads kb's buffer any more, so the second
  // stage refills it with K block kb+2 while reading K block kb+1's first
  // fragments and scales.  One barrier per K block.
  // kblock(p, kb, ...): K block kb in buffer p with scale set (csa, csb);
  // dma: load K block kb+2; next: kb+1 exists (read its scales into (nsa, nsb)).
  // sg: also load scale group (kb >> 2) + 1 (kb = 0 mod 4: the first K block
  // of each four, and of a trailing pair).  The group lands in its area,
  // whose previous group was last read one K block earlier; a group past the
  // last K block loads clamped bytes nobody reads.  A group is read from 3 to
  // 6 K blocks later on.
  auto kblock = [&](int p, int kb, bool dma, bool next, bool sg, const int (&csa)[MT], const int (&csb)[NT * SBP],
                    int (&nsa)[MT], int (&nsb)[NT * SBP]) __attribute__((always_inline)) {
    stage(0, -1, 0, p, 1, false, 0, -1, fa0, fb0, fa1, fb1, csa, csb, nsa, nsb);
    if (dma || next) wait_vm_barrier<0>();
    stage(1, dma ? p : -1, kb + 2, next ? (p ^ 1) : -1, 0, next, kb + 1, sg ? (kb >> 2) + 1 : -1, fa1, fb1, fa0,
          fb0, csa, csb, nsa, nsb);
  };

  // ---- prologue: K blocks 0 and 1 in flight, then K block 0's first
  // fragments and scales.  K block kb sits in buffer kb % 2.
  if (nkb > 0) {
    sdma_group(0);
    dma_kblock(0, 0);
    if (nkb > 1) {
      dma_kblock(1, 1);
      wait_vm_barrier<DMA_ITEMS>();
    } else {
      wait_vm_barrier<0>();
    }
    read_frags(0, 0, fa0, fb0);
    read_scales(0, sa0, sb0);
  }

  // ---- steady state: K blocks whose second stage loads a later block, in
  // fours (one scale group load each: a loop of pairs loading the group in
  // every pair spent 10 % more load instructions and ran 1-3 % slower), then
  // a pair and a lone one as their count needs.  The loop body names its
  // buffers as constants and every path into the loop has the same loads in
  // flight, so the compiler's per-buffer tracking of in-flight LDS-bound
  // loads stays exact around it.
  const int main_kb = nkb - 2;  // K blocks whose second stage loads a later block
  int kb = 0;
#pragma nounroll
  for (; kb + 3 < main_kb; kb += 4) {  // four K blocks: buffers 0, 1, 0, 1; scale sets 0, 1, 0, 1
    kblock(0, kb, true, true, true, sa0, sb0, sa1, sb1);
    kblock(1, kb + 1, true, true, false, sa1, sb1, sa0, sb0);
    kblock(0, kb + 2, true, true, false, sa0, sb0, sa1, sb1);
    kblock(1, kb + 3, true, true, false, sa1, sb1, sa0, sb0);
  }
  if (kb + 1 < main_kb) {
    kblock(0, kb, true, true, true, sa0, sb0, sa1, sb1);
    kblock(1, kb + 1, true, true, false, sa1, sb1, sa0, sb0);
    kb += 2;
  }
  if (kb < main_kb) {
    kblock(0, kb, true, true, false, sa0, sb0, sa1, sb1);
    // The drain takes K block kb + 1's scales from set 0; with F32S set 1
    // must then hold K block kb's (its temporaries are added in the drain).
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int t = sa0[mt];
      sa0[mt] = sa1[mt];
      if (F32S) sa1[mt] = t;
    }
#pragma unroll
    for (int i = 0; i < NT * SBP; ++i) {
      const int t = sb0[i];
      sb0[i] = sb1[i];
      if (F32S) sb1[i] = t;
    }
  }

  // Pins the accumulators to AGPRs where the K loop ends: left free, the
  // allocator moves some of them into VGPRs during the drain (the epilogue
  // reads them through VALU) and spills fragments to make room.
  auto pin_acc = [&]() __attribute__((always_inline)) {
    if constexpr (!F32S) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+a"(acc[mt][nt]));
    }
  };
  // F32S: the last K block's temporaries, after the retire pad.
  auto apply_all = [&](const int (&ps_a)[MT], const int (&ps_b)[NT * SBP]) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) apply(mt, nt, ps_a, ps_b);
  };

  // ---- epilogue.  Lane l holds, for each (mt, nt), C[r][c .. c+3] with
  // r = l & 31 and c = 8q + 4(l >> 5) (q = 0..3) inside the 32x32 block.
  // Stored from registers directly, that is 16 rows x 16 bytes per store
  // instruction.  Instead each wave stages one 32-row strip of its
  // sub-tile at a time in LDS and writes it back row by row: every store
  // instruction then covers whole 256-byte row segments.  The stores are
  // non-temporal: output lines are written once, and kept out of L2 they
  // leave the operand tiles other workgroups still read in place (measured:
  // 5 % on the fprop shape, none lost elsewhere).  The staging sits in one
  // K-block buffer nothing reads any more, each wave in its own 32-row region
  // (stage_buf + wave * 32 * P); only the wave itself touches its region, and
  // LDS executes one wave's accesses in order, so no barrier is needed.
  auto epilogue = [&](uint8_t* stage_buf) __attribute__((always_inline)) {
    if (!out_bf16) {
      // Unpadded rows, the 16-byte chunk c of row r at chunk c ^ (r & 15):
      // the 16 rows a write instruction's lane group covers land in 16
      // different chunks, and a read covers whole rows.  (Without a pad the
      // 128x128 tile's LDS is 80 KB, two workgroups per compute unit.)
      constexpr int P = WN * 4;  // bytes per staged row
      static_assert(4 * 32 * P <= PB, "staging fits a buffer");
      uint8_t* stg = stage_buf + wave * (32 * P);
      constexpr int CH = WN / 4;            // 16-byte chunks per row
      static_assert(CH >= 16, "swizzle within a row");
      constexpr int ROWS_PER = 64 / CH;     // rows per store instruction
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        __builtin_amdgcn_sched_barrier(0);  // one strip's accumulators at a time
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v4f v = v4f{acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1], acc[mt][nt][4 * q + 2],
                              acc[mt][nt][4 * q + 3]};
            *reinterpret_cast<v4f*>(stg + (lane & 31) * P + (((nt * 8 + 2 * q + g) ^ (lane & 15)) * 16)) = v;
          }
        const int row0 = m0 + wm * WM + mt * 32;
#pragma unroll
        for (int it = 0; it < 32 / ROWS_PER; ++it) {
          const int rr = it * ROWS_PER + lane / CH, ch = lane % CH;
          const v4f v = *reinterpret_cast<const v4f*>(stg + rr * P + ((ch ^ (rr & 15)) * 16));
          const int m = row0 + rr, n = n0 + wn * WN + ch * 4;
          if (m < M) {
            float* dst = reinterpret_cast<float*>(C) + (int64_t)m * ldc + n;
            if (n + 3 < N) {
              __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(dst));
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (n + i < N) dst[i] = v[i];
            }
          }
        }
      }
    } else {
      constexpr int P = WN * 2 + 16;
      uint8_t* stg = stage_buf + wave * (32 * P);
      constexpr int CH = WN / 8;
      constexpr int ROWS_PER = 64 / CH;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        __builtin_amdgcn_sched_barrier(0);  // one strip's accumulators at a time
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint2 o;
            o.x = bf16x2_rne(acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1]);
            o.y = bf16x2_rne(acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]);
            *reinterpret_cast<uint2*>(stg + (lane & 31) * P + (nt * 32 + 8 * q + 4 * g) * 2) = o;
          }
        const int row0 = m0 + wm * WM + mt * 32;
#pragma unroll
        for (int it = 0; it < 32 / ROWS_PER; ++it) {
          const int rr = it * ROWS_PER + lane / CH, ch = lane % CH;
          const uint4 v = *reinterpret_cast<const uint4*>(stg + rr * P + ch * 16);
          const int m = row0 + rr, n = n0 + wn * WN + ch * 8;
          if (m < M) {
            uint16_t* dst = reinterpret_cast<uint16_t*>(C) + (int64_t)m * ldc + n;
            if (n + 7 < N) {
              __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
            } else {
              const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
              for (int i = 0; i < 8; ++i)
                if (n + i < N) dst[i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
            }
          }
        }
      }
    }
  };

  // ---- drain: the last (up to) two K blocks, no further loads; then the
  // epilogue.  Their buffers depend on the parity of the K block count and
  // are chosen at run time here (this costs a full wait for the last load
  // before the drain's first LDS read, once per tile).  Each exit path has
  // its own epilogue, in a buffer nobody reads after the drain's barrier.
  if (nkb >= 2) {
    const int p = nkb & 1;  // buffer of K block nkb - 2
    kblock(p, nkb - 2, false, true, false, sa0, sb0, sa1, sb1);
    kblock(p ^ 1, nkb - 1, false, false, false, sa1, sb1, sa0, sb0);
    mfma_retire_pad();
    apply_all(sa1, sb1);
    pin_acc();
    epilogue(buf_ptr(p));
  } else if (BM < 256 && nkb == 1) {  // the 256-wide tile is launched with K >= 256 only
    kblock(0, 0, false, false, false, sa0, sb0, sa1, sb1);
    mfma_retire_pad();
    apply_all(sa0, sb0);
    pin_acc();
    epilogue(kbuf1);  // never loaded when K = 128
  } else if (BM < 256) {
    epilogue(kbuf0);  // K = 0: zeros
  }
#endif
}

// The 128x128 tile (80 KB of LDS, at most 256 registers) runs two
// workgroups per compute unit; the others one.  With fp32 scales per column
// of B (16 scale values per fragment) 256 registers make the K loop spill,
// so that variant keeps one.
template <int BM, int BN, int STAGES, int AFMT, int BFMT, bool BKN, bool BROW, bool MXS, bool F32S, bool WS>
__global__ __launch_bounds__(kThreads, (BM == 128 && !(F32S && BROW)) ? 2 : 1) void gemm_bs_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ SA,
    const uint8_t* __restrict__ B, int64_t ldb, const uint8_t* __restrict__ SB, void* __restrict__ C,
    int64_t ldc, int out_bf16, int tiles_m, int tiles_n, int tile_first) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef TileLds<BM, BN> L;
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[L::PB];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[L::PB];
  __shared__ __attribute__((aligned(1024))) uint8_t sgrp[L::SGRP];
  gemm_tile<BM, BN, STAGES, AFMT, BFMT, BKN, BROW, MXS, F32S, WS>(M, N, K, A, lda, SA, B, ldb, SB, C, ldc,
                                                                 out_bf16, tiles_m, tiles_n, tile_first, 0, 0,
                                                                 blockIdx.x, gridDim.x, kbuf0, kbuf1, sgrp);
#endif
}

// The cells past the last full round of 256x256 tiles as 128x128 quadrants
// (kTailSub workgroups per cell, workgroups 0 .. nq - 1), then cells
// 0 .. big - 1 as 256x256 tiles (workgroups nq ..), in one launch.
// Workgroups start in id order as compute units free up: the quadrants run
// first on most compute units while the rest start 256x256 tiles, so the
// compute units reach their epilogues at two different times and each
// burst of output stores is smaller.  Quadrants last, the whole chip wrote
// its tiles at once, twice, and 64 compute units sat idle in the quadrant
// round: 4096x8960x1536 took 60.7-61.5 us (bf16 out) and 71.6-72.2 us
// (fp32 out) that way against 56.2-58.7 and 63.3-65.6 us now,
// 4096x8960x4096 129.5-130.1 against 120.6-121.3 us (A/B in one process).
// big is a multiple of 8 and the 256x256 part's ids are offset by the
// constant nq, which only permutes the XCDs, so it keeps its per-XCD bands.
// (256x128 halves instead of quadrants, half as many workgroups, took 3 us
// longer on the 4096x8960x1536 shape.)
constexpr int kTailSub = 4;
template <int AFMT, int BFMT, bool BKN, bool BROW, bool MXS, bool WS>
__global__ __launch_bounds__(kThreads, 1) void gemm_bs_split_tail_kernel(
    int M, int N, int K, const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ SA,
    const uint8_t* __restrict__ B, int64_t ldb, const uint8_t* __restrict__ SB, void* __restrict__ C,
    int64_t ldc, int out_bf16, int tiles_m, int tiles_n, int big) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef TileLds<256, 256> L;
  static_assert(TileLds<128, 128>::PB <= L::PB && TileLds<128, 128>::SGRP <= L::SGRP, "quadrant LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[L::PB];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[L::PB];
  __shared__ __attribute__((aligned(1024))) uint8_t sgrp[L::SGRP];
  const int nq = (int)gridDim.x - big;
  const int b = blockIdx.x;
  if (b >= nq)
    gemm_tile<256, 256, 4, AFMT, BFMT, BKN, BROW, MXS, false, WS>(M, N, K, A, lda, SA, B, ldb, SB, C, ldc,
                                                                  out_bf16, tiles_m, tiles_n, 0, 0, 0, b - nq, big,
                                                                  kbuf0, kbuf1, sgrp);
  else
    gemm_tile<128, 128, 4, AFMT, BFMT, BKN, BROW, MXS, false, WS>(M, N, K, A, lda, SA, B, ldb, SB, C, ldc,
                                                                  out_bf16, tiles_m, tiles_n, big, 1, 1, b, nq,
                                                                  kbuf0, kbuf1, sgrp);
#endif
}

template <int BM, int BN, int STAGES, int AFMT, int BFMT, bool BKN, bool BROW, bool MXS, bool F32S, bool WS>
void launch_tile(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa,
                 const uint8_t* b, int64_t ldb, const uint8_t* sb, void* c, int64_t ldc, int c_dtype,
                 int tiles_m, int tiles_n, int tile_first, int cells, hipStream_t stream) {
  if (cells <= 0) return;
  hipLaunchKernelGGL((gemm_bs_kernel<BM, BN, STAGES, AFMT, BFMT, BKN, BROW, MXS, F32S, WS>), dim3(cells),
                     dim3(kThreads), 0, stream, (int)M, (int)N, (int)K, a, lda, sa, b, ldb, sb, c, ldc,
                     c_dtype == 1 ? 1 : 0, tiles_m, tiles_n, tile_first);
}

// Tile choice: 128x128 when its tiles fit on the CUs at two per CU (one
// round), else 256x256 (128x128 per wave, the lowest LDS traffic per MFMA);
// a short last round of 256x256 tiles runs as 128x128 quadrants.  Measured
// at M = 4096 (K = 4096): N = 2048 (512 small tiles) 34 us against 43 us for
// 256x256, N = 2560 (640 small tiles, two rounds of them) 55 against 44 us.
// Building with -DMXFP8_GEMM_TILE=128 or 256 pins one tile size everywhere
// (for tuning).
#ifndef MXFP8_GEMM_TILE
#define MXFP8_GEMM_TILE 0
#endif
template <int AFMT, int BFMT, bool BKN, bool BROW, bool MXS, bool WS>
void launch_shape(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa,
                  const uint8_t* b, int64_t ldb, const uint8_t* sb, void* c, int64_t ldc, int c_dtype,
                  hipStream_t stream) {
  const int bm = (int)((M + 255) / 256), bn = (int)((N + 255) / 256), big_tiles = bm * bn;
  const int sm = (int)((M + 127) / 128), sn = (int)((N + 127) / 128);
  const int cus = device_cus();
  // The 256-wide tile needs K >= 256: a separate single-K-block drain would
  // make the accumulators spill (merging three exit paths of 256 of them).
  const bool big = K >= 256 && (MXFP8_GEMM_TILE == 256 || (MXFP8_GEMM_TILE == 0 && sm * sn > 2 * cus));
  if (!big) {
    launch_tile<128, 128, 4, AFMT, BFMT, BKN, BROW, MXS, false, WS>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype,
                                                                   sm, sn, 0, sm * sn, stream);
    return;
  }
  // Last partial round: when its 256x256 tiles, cut in kTailSub, fit on the
  // CUs in one round of sub-tiles, that round takes a fraction as long.
  const int tail = big_tiles % cus;
  const bool split_tail = MXFP8_GEMM_TILE == 0 && big_tiles > cus && tail > 0 && kTailSub * tail <= cus;
  if (!split_tail) {
    launch_tile<256, 256, 4, AFMT, BFMT, BKN, BROW, MXS, false, WS>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype,
                                                                   bm, bn, 0, big_tiles, stream);
    return;
  }
  // main_cells is a multiple of the CU count (256 = 8 XCDs x 32), so both
  // parts of the launch keep their per-XCD bands.
  const int main_cells = big_tiles - tail;
  hipLaunchKernelGGL((gemm_bs_split_tail_kernel<AFMT, BFMT, BKN, BROW, MXS, WS>), dim3(main_cells + kTailSub * tail),
                     dim3(kThreads), 0, stream, (int)M, (int)N, (int)K, a, lda, sa, b, ldb, sb, c, ldc,
                     c_dtype == 1 ? 1 : 0, bm, bn, main_cells);
}

template <int AFMT, int BFMT>
void launch_fmt(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa,
                const uint8_t* b, int64_t ldb, int b_layout, const uint8_t* sb, int b_scale_mode, void* c,
                int64_t ldc, int c_dtype, hipStream_t stream) {
  // Wide scale loads (one 4-byte load per row for 4 K blocks) need 4-byte
  // aligned rows: K blocks a multiple of 4 and 4-byte aligned row scales.
  const int64_t nkb = K / 128;
  const bool brow = b_layout == 0 && b_scale_mode == 1;
  const bool ws = nkb >= 4 && nkb % 4 == 0 && reinterpret_cast<uintptr_t>(sa) % 4 == 0 &&
                  (!brow || reinterpret_cast<uintptr_t>(sb) % 4 == 0);
#define MXFP8_SHAPE(BKN, BROW)                                                                                \
  (ws ? launch_shape<AFMT, BFMT, BKN, BROW, false, true>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype, stream) \
      : launch_shape<AFMT, BFMT, BKN, BROW, false, false>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype, stream))
  if (b_layout == 1)
    MXFP8_SHAPE(true, false);
  else if (brow)
    MXFP8_SHAPE(false, true);
  else
    MXFP8_SHAPE(false, false);
#undef MXFP8_SHAPE
}

// fp32 block scales: 128x128 tiles only (the temporaries double the
// accumulator registers).
template <int AFMT, int BFMT>
void launch_f32s_fmt(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa,
                     const uint8_t* b, int64_t ldb, int b_layout, const uint8_t* sb, int b_scale_mode, void* c,
                     int64_t ldc, int c_dtype, hipStream_t stream) {
  const int sm = (int)((M + 127) / 128), sn = (int)((N + 127) / 128);
  if (b_layout == 1)
    launch_tile<128, 128, 4, AFMT, BFMT, true, false, false, true, false>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype,
                                                                  sm, sn, 0, sm * sn, stream);
  else if (b_scale_mode == 1)
    launch_tile<128, 128, 4, AFMT, BFMT, false, true, false, true, false>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype,
                                                                  sm, sn, 0, sm * sn, stream);
  else
    launch_tile<128, 128, 4, AFMT, BFMT, false, false, false, true, false>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc,
                                                                   c_dtype, sm, sn, 0, sm * sn, stream);
}

template <int AFMT, int BFMT>
void launch_mx_fmt(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa,
                   const uint8_t* b, int64_t ldb, const uint8_t* sb, void* c, int64_t ldc, int c_dtype,
                   hipStream_t stream) {
  launch_shape<AFMT, BFMT, false, true, true, false>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype, stream);
}

#define MXFP8_GEMM_PAIR(AF, BF)                                                                                   \
  template void launch_fmt<AF, BF>(int64_t, int64_t, int64_t, const uint8_t*, int64_t, const uint8_t*,            \
                                   const uint8_t*, int64_t, int, const uint8_t*, int, void*, int64_t, int,         \
                                   hipStream_t);                                                                   \
  template void launch_f32s_fmt<AF, BF>(int64_t, int64_t, int64_t, const uint8_t*, int64_t, const uint8_t*,       \
                                        const uint8_t*, int64_t, int, const uint8_t*, int, void*, int64_t, int,    \
                                        hipStream_t);                                                              \
  template void launch_mx_fmt<AF, BF>(int64_t, int64_t, int64_t, const uint8_t*, int64_t, const uint8_t*,         \
                                      const uint8_t*, int64_t, const uint8_t*, void*, int64_t, int, hipStream_t);
#if MXFP8_GEMM_FMT == 4
MXFP8_GEMM_PAIR(0, 0)
MXFP8_GEMM_PAIR(1, 0)
MXFP8_GEMM_PAIR(0, 1)
MXFP8_GEMM_PAIR(1, 1)
#else
MXFP8_GEMM_PAIR((MXFP8_GEMM_FMT >> 1), (MXFP8_GEMM_FMT & 1))
#endif
#undef MXFP8_GEMM_PAIR

#endif  // MXFP8_GEMM_FMT >= 0

}  // namespace gemm_detail

using namespace gemm_detail;

#if MXFP8_GEMM_FMT == 4 || MXFP8_GEMM_FMT < 0

void launch_gemm_f32s(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, int a_fmt,
                      const float* sa, const uint8_t* b, int64_t ldb, int b_fmt, int b_layout, const float* sb,
                      int b_scale_mode, void* c, int64_t ldc, int c_dtype, hipStream_t stream) {
  const uint8_t* sa8 = reinterpret_cast<const uint8_t*>(sa);
  const uint8_t* sb8 = reinterpret_cast<const uint8_t*>(sb);
  if (a_fmt == 0 && b_fmt == 0)
    launch_f32s_fmt<0, 0>(M, N, K, a, lda, sa8, b, ldb, b_layout, sb8, b_scale_mode, c, ldc, c_dtype, stream);
  else if (a_fmt == 1 && b_fmt == 0)
    launch_f32s_fmt<1, 0>(M, N, K, a, lda, sa8, b, ldb, b_layout, sb8, b_scale_mode, c, ldc, c_dtype, stream);
  else if (a_fmt == 0 && b_fmt == 1)
    launch_f32s_fmt<0, 1>(M, N, K, a, lda, sa8, b, ldb, b_layout, sb8, b_scale_mode, c, ldc, c_dtype, stream);
  else
    launch_f32s_fmt<1, 1>(M, N, K, a, lda, sa8, b, ldb, b_layout, sb8, b_scale_mode, c, ldc, c_dtype, stream);
}

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

void launch_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, int a_fmt,
                    const uint8_t* sa, const uint8_t* b, int64_t ldb, int b_fmt, const uint8_t* sb, void* c,
                    int64_t ldc, int c_dtype, hipStream_t stream) {
  if (a_fmt == 0 && b_fmt == 0)
    launch_mx_fmt<0, 0>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype, stream);
  else if (a_fmt == 1 && b_fmt == 0)
    launch_mx_fmt<1, 0>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype, stream);
  else if (a_fmt == 0 && b_fmt == 1)
    launch_mx_fmt<0, 1>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype, stream);
  else
    launch_mx_fmt<1, 1>(M, N, K, a, lda, sa, b, ldb, sb, c, ldc, c_dtype, stream);
}

#endif  // host dispatch

}  // namespace mxfp8
