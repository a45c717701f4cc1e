/*
 * mxfp8.h -- C ABI of libmxfp8: hybrid-granularity FP8 quantization with
 * power-of-two (E8M0) scales, and the block-scaled FP8 GEMM that consumes it,
 * for AMD Instinct MI355X (gfx950).  Next to them: the MX GEMM on 32-element
 * scales, two-orientation quantizers, an fp32-scale variant of the quantizers
 * and the GEMM, and the GaussWS weight sampler.
 *
 * Sources (web pages, cited by title and section):
 *   [FP8F] "FP8 Formats for Deep Learning", review page, "Core claim": the
 *          E4M3 and E5M2 encodings (E4M3 without infinities and with one NaN
 *          pattern, E5M2 with IEEE 754 specials).
 *   [INFR] "A Comprehensive FP8 Training Recipe for Reasoning-Enhanced
 *          Language Models", review page, "What carries the argument" and
 *          Figs. 1-2: per-token scales for activations and gradients,
 *          per-block scales for weights, UE8M0 scales rounded up to a power
 *          of two so the scaled tensor never leaves the FP8 range, FP8
 *          forward and backward GEMMs.
 *   [MXTI] "Characterization and Mitigation of Training Instabilities in
 *          Microscaling Formats", review page, "What carries the argument"
 *          and Fig. 5: 32-element MX blocks sharing one E8M0 scale, the
 *          clamping of scaled values above the largest code, and a monitor
 *          of the clamped fraction ("Reading between the lines").
 *   [GWS]  "Gaussian Weight Sampling for Scalable, Efficient and Stable
 *          Pseudo-Quantization Training", review page, "The reading" and
 *          "What carries the argument": the sampled weight
 *          w + R * max_bl(|w|) * 2^(1 - b_t) with rounded-normal R and a
 *          bitwidth b_t per 32x32 block, cast to BF16.
 *
 * Conventions shared by every entry point
 *   - Pointers to tensors are DEVICE pointers owned by the caller; the
 *     library never allocates, frees, or synchronizes.  Work is enqueued
 *     asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 *   - All tensors are row-major with an explicit leading dimension `ld*`
 *     counted in ELEMENTS of that tensor.  Scale and count arrays are dense
 *     (no leading dimension).  A scale byte b stands for 2^(b - 127).
 *   - Inputs are never written; outputs are overwritten in full (codes
 *     beyond the logical width of a row, up to `ld`, are not touched).
 *   - Alignment: every code or value tensor pointer is 16-byte aligned and
 *     every `ld` is a multiple of 16 elements (MXFP8_ERR_ALIGN /
 *     MXFP8_ERR_LD otherwise).  Byte scale arrays need no alignment; scale
 *     arrays read as 32-bit words (fp32 scales, mx_gemm's scales) are 4-byte
 *     aligned.
 *   - Outputs must not share an address with an input (MXFP8_ERR_ALIAS,
 *     checked by pointer equality; partial overlap is undefined).
 *   - Empty problems (a zero extent) return MXFP8_OK without launching, and
 *     their pointers may then be NULL.
 *   - The return value reports host-side argument validation (checked before
 *     any HIP call, so it is usable without a GPU) and launch errors
 *     (MXFP8_ERR_DEVICE wraps hipGetLastError).  Device-side results are
 *     only defined after the stream has been synchronized.
 *   - Non-finite input values are outside the contract (no fault; the bytes
 *     produced are unspecified).
 *   - Casts are round-to-nearest, ties to even, saturating at the largest
 *     finite value (448 for E4M3, 57344 for E5M2); the sign of zero is kept.
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXFP8_VERSION 100 /* 1.0.0 */

typedef enum {
  MXFP8_OK = 0,
  MXFP8_ERR_NULL = 1,   /* a required pointer is NULL */
  MXFP8_ERR_SHAPE = 2,  /* negative extent or extent not allowed by the entry point */
  MXFP8_ERR_LD = 3,     /* leading dimension smaller than the row or not a multiple of 16 */
  MXFP8_ERR_ALIGN = 4,  /* a tensor pointer is not 16-byte aligned */
  MXFP8_ERR_ENUM = 5,   /* an enum argument is out of range or an unsupported combination */
  MXFP8_ERR_ALIAS = 6,  /* an output pointer equals an input pointer */
  MXFP8_ERR_DEVICE = 7  /* the HIP runtime reported an error at launch */
} mxfp8_status;

typedef enum { MXFP8_E4M3 = 0, MXFP8_E5M2 = 1 } mxfp8_fmt; /* OCP encodings [FP8F] */
typedef enum { MXFP8_F32 = 0, MXFP8_BF16 = 1 } mxfp8_dtype;
typedef enum { MXFP8_GROUP_ROW = 0, MXFP8_GROUP_COL_T = 1 } mxfp8_axis;
typedef enum { MXFP8_RULE_CEIL = 0, MXFP8_RULE_FLOOR = 1 } mxfp8_rule;
typedef enum { MXFP8_B_NK = 0, MXFP8_B_KN = 1 } mxfp8_blayout;
typedef enum { MXFP8_SCALE_BLOCK128 = 0, MXFP8_SCALE_ROW128 = 1 } mxfp8_bscale;

/*
 * fp8_quantize_token -- token-wise 1x128 quantization of activations or
 * gradients [INFR "What carries the argument", Fig. 2].
 *
 * x: [rows][ldx] of fp32 or bf16 (x_dtype), logical width `cols`.
 * For each group of up to 128 consecutive elements along `axis`:
 *   amax = max |x| over the group;
 *   e    = the smallest integer with amax <= fmax * 2^e, clamped to
 *          [-127, 127] (amax == 0 gives -127): the round-up power of two;
 *   scale byte = e + 127;  code = cast(x * 2^-e)  (never saturates).
 *
 * axis == MXFP8_GROUP_ROW: groups run along each row (cols).
 *   q:      [rows][ldq >= cols] codes, same layout as x.
 *   scales: [rows][ceil(cols / 128)].
 *   Requires cols % 16 == 0 (the last group of a row may hold 16..112).
 * axis == MXFP8_GROUP_COL_T: groups run down each column (128 consecutive
 *   rows = tokens), and codes are written transposed so that the token axis
 *   is contiguous (the operand layout of a weight-gradient GEMM whose K is
 *   the token axis).
 *   q:      [cols][ldq >= rows] codes (q[c * ldq + r] encodes x[r][c]).
 *   scales: [cols][ceil(rows / 128)].
 *   Requires rows % 16 == 0 and cols % 16 == 0.
 */
int fp8_quantize_token(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                       int axis, int fmt, uint8_t* q, int64_t ldq, uint8_t* scales,
                       void* stream);

/*
 * fp8_quantize_block -- block-wise 128x128 quantization of weights
 * [INFR "What carries the argument", Fig. 1].
 *
 * w: [rows][ldw] of fp32 or bf16, logical width `cols`.  One round-up scale
 * (as above) per 128x128 tile, tiles at the right and bottom edges partial.
 *   q:      [rows][ldq >= cols] codes, same layout as w.
 *   scales: [ceil(rows / 128)][ceil(cols / 128)].
 * Requires cols % 16 == 0.  A square tile has the same scale for w and its
 * transpose, so the same codes serve a GEMM reading w as [N][K] or [K][N].
 */
int fp8_quantize_block(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ldw,
                       int fmt, uint8_t* q, int64_t ldq, uint8_t* scales, void* stream);

/*
 * fp8_quantize_token_f32s, fp8_quantize_block_f32s -- the token-wise and the
 * block-wise quantizers with fp32 scales instead of power-of-two bytes: the
 * "FP8 w. FP32 scale" variant that the recipe's Table 4 compares [INFR, review
 * page, the referee's minor comment on Section 5.2.1, which names it; the page
 * does not define it, so it is read here as ordinary fp32 scaling]:
 *   s    = amax / fmax in IEEE fp32 (round to nearest even); s = 1 where
 *          that quotient is zero (amax == 0, or amax < fmax * 2^-150);
 *   code = cast(x / s), the fp32 quotient cast with round-to-nearest-even,
 *          saturating at +-fmax (the rounding of s can put a quotient a
 *          little above fmax).
 * Arguments, groups, layouts and requirements are those of
 * fp8_quantize_token and fp8_quantize_block, with `scales` an array of fp32
 * (4-byte aligned, MXFP8_ERR_ALIGN otherwise) in the same layout.  A value is
 * recovered as dec(code) * s.
 */
int fp8_quantize_token_f32s(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                            int axis, int fmt, uint8_t* q, int64_t ldq, float* scales, void* stream);
int fp8_quantize_block_f32s(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ldw,
                            int fmt, uint8_t* q, int64_t ldq, float* scales, void* stream);

/*
 * fp8_quantize_token_dual -- both orientations of fp8_quantize_token from one
 * read of x: the ROW groups that the forward GEMM consumes and the transposed
 * COL_T groups that the weight-gradient GEMM consumes [INFR "What carries the
 * argument", Fig. 2: one tensor quantized token-wise feeds the forward and
 * the backward GEMMs].  The outputs are byte-for-byte those of the two
 * one-orientation calls:
 *   q:        [rows][ldq >= cols],  scales:   [rows][ceil(cols / 128)]  (ROW);
 *   qt:       [cols][ldqt >= rows], scales_t: [cols][ceil(rows / 128)]  (COL_T).
 * Requires rows % 16 == 0 and cols % 16 == 0; the four outputs are distinct.
 */
int fp8_quantize_token_dual(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                            int fmt, uint8_t* q, int64_t ldq, uint8_t* scales, uint8_t* qt,
                            int64_t ldqt, uint8_t* scales_t, void* stream);

/*
 * fp8_quantize_block_dual -- fp8_quantize_block plus the transposed codes
 * [INFR "What carries the argument", Fig. 1: 128x128 weight blocks serve the
 * forward and the input-gradient GEMMs].  A tile has one scale, so its
 * transpose holds the same bytes:
 *   q:        [rows][ldq >= cols],  scales:   [ceil(rows/128)][ceil(cols/128)];
 *   qt:       [cols][ldqt >= rows], scales_t: [ceil(cols/128)][ceil(rows/128)]
 *             (qt[c * ldqt + r] = q[r * ldq + c]; scales_t is scales
 *             transposed), so a GEMM can read w^T as an [N][K] operand with
 *             MXFP8_SCALE_BLOCK128 scales.
 * Requires rows % 16 == 0 and cols % 16 == 0; the four outputs are distinct.
 */
int fp8_quantize_block_dual(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ldw,
                            int fmt, uint8_t* q, int64_t ldq, uint8_t* scales, uint8_t* qt,
                            int64_t ldqt, uint8_t* scales_t, void* stream);

/*
 * mx_quantize -- MX quantization, 32 consecutive elements of a row sharing
 * one E8M0 scale [MXTI "What carries the argument", Fig. 5].
 *
 * rule == MXFP8_RULE_FLOOR (the OCP MX rule):
 *   X = floor(log2 amax) - emax_elem, emax_elem = 8 (E4M3) or 15 (E5M2),
 *   clamped to [-127, 127] (amax == 0 gives -127).  Scaled values can exceed
 *   fmax (the scaled amax lies in [256, 512) for E4M3) and then saturate to
 *   the largest code: the last-bin clamping the MX page describes.
 * rule == MXFP8_RULE_CEIL: the round-up scale of fp8_quantize_token.
 *   q:            [rows][ldq >= cols] codes.
 *   scales:       [rows][cols / 32], byte X + 127.
 *   clamp_counts: NULL, or [rows][cols / 32]: per block, the number of
 *                 elements with |x| * 2^-X > fmax (0..32).
 * Requires cols % 32 == 0.
 */
int mx_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                int rule, uint8_t* q, int64_t ldq, uint8_t* scales, uint8_t* clamp_counts,
                void* stream);

/*
 * fp8_block_scaled_gemm -- C = A * B over dequantized FP8 operands with
 * fp32 accumulation [INFR "What carries the argument": FP8 GEMMs on
 * per-token / per-block scaled operands]:
 *
 *   C[m][n] = sum over 128-wide K blocks kb of
 *             2^(sa(m,kb) - 127) * 2^(sb(kb,n) - 127) *
 *             sum_{k in kb} dec(A[m][k]) * dec(B(k, n)).
 *
 * a:        [M][lda >= K] codes (a_fmt), K contiguous.
 * a_scales: [M][K / 128] (the layout fp8_quantize_token ROW produces).
 * b:        b_layout == MXFP8_B_NK: [N][ldb >= K] (K contiguous);
 *           b_layout == MXFP8_B_KN: [K][ldb >= N] (N contiguous).
 * b_scales: b_scale_mode == MXFP8_SCALE_BLOCK128: one byte per 128x128 tile
 *             of B's storage: NK -> [ceil(N/128)][K/128],
 *             KN -> [K/128][ceil(N/128)] (fp8_quantize_block's layout);
 *           b_scale_mode == MXFP8_SCALE_ROW128 (NK only): [N][K / 128]
 *             (fp8_quantize_token's layout, e.g. for the weight gradient).
 * c:        [M][ldc >= N], fp32 or bf16 (c_dtype; bf16 is rounded to
 *           nearest even once, from the fp32 accumulator).  Overwritten.
 * Requires K % 128 == 0 and lda, ldb <= 2^24 (MXFP8_ERR_LD otherwise: the
 * kernels address a tile with 32-bit offsets); M and N are arbitrary
 * (partial edge tiles).
 * Accuracy: fp32 accumulation of 64-wide matrix-core partial sums, plus one
 * bf16 rounding when c_dtype is bf16.  The matrix cores add the products of
 * each run of 8 consecutive k after aligning them to the run's largest
 * exponent sum E and truncating below 2^(E-13): operands quantized from real
 * tensors stay within 2^-12 * sum_k |a_mk * b_kn| of the exact sum; operands
 * whose products in one run span many binades (arbitrary codes) can lose up
 * to 8 * 2^(E-13) * scale per run.
 */
int fp8_block_scaled_gemm(int64_t M, int64_t N, int64_t K,
                          const uint8_t* a, int64_t lda, int a_fmt, const uint8_t* a_scales,
                          const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
                          const uint8_t* b_scales, int b_scale_mode,
                          void* c, int64_t ldc, int c_dtype, void* stream);

/*
 * fp8_gemm_f32s -- fp8_block_scaled_gemm over operands with fp32 scales (the
 * output of fp8_quantize_token_f32s / fp8_quantize_block_f32s; the "FP8 w.
 * FP32 scale" variant, see those):
 *
 *   C[m][n] = sum over 128-wide K blocks kb of
 *             sa(m,kb) * sb(kb,n) * sum_{k in kb} dec(A[m][k]) * dec(B(k, n)).
 *
 * Arguments, layouts and requirements are those of fp8_block_scaled_gemm,
 * with a_scales and b_scales arrays of fp32 (4-byte aligned) in the same
 * layouts.  Each K block's product is accumulated by the matrix cores in
 * fp32 (with the alignment described for fp8_block_scaled_gemm) and added
 * into the fp32 result times fl(sa * sb) with one fused multiply-add (per-
 * column B scales: times fl(sa * sb(n))); the scale product's rounding adds at
 * most 2^-23 * sum_k |a_mk * b_kn| to the bound of fp8_block_scaled_gemm.
 * Runs on 128x128 tiles.
 */
int fp8_gemm_f32s(int64_t M, int64_t N, int64_t K,
                  const uint8_t* a, int64_t lda, int a_fmt, const float* a_scales,
                  const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
                  const float* b_scales, int b_scale_mode,
                  void* c, int64_t ldc, int c_dtype, void* stream);

/*
 * mx_gemm -- C = A * B over MX operands: FP8 elements with one E8M0 scale
 * per 32 consecutive elements along K, fp32 accumulation [MXTI "What carries
 * the argument": the matrix products of MX training run on operands whose
 * 32-element blocks share one power-of-two scale]:
 *
 *   C[m][n] = sum over 32-wide K blocks j of
 *             2^(sa[m][j] - 127) * 2^(sb[n][j] - 127) *
 *             sum_{k in j} dec(A[m][k]) * dec(B[n][k]).
 *
 * a:        [M][lda >= K] codes (a_fmt), K contiguous.
 * a_scales: [M][K / 32] (mx_quantize's scale layout for A's rows).
 * b:        [N][ldb >= K] codes (b_fmt), K contiguous (B stored as B^T,
 *           e.g. a weight [out][in] quantized along its rows by mx_quantize).
 * b_scales: [N][K / 32].
 * c:        [M][ldc >= N], fp32 or bf16 (c_dtype), overwritten.
 * Requires K % 128 == 0 and 4-byte aligned scale pointers (plus the
 * alignment and leading-dimension rules of fp8_block_scaled_gemm, lda and
 * ldb <= 2^24 included); M and N are arbitrary.  Accuracy as for
 * fp8_block_scaled_gemm.
 */
int mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, int a_fmt,
            const uint8_t* a_scales, const uint8_t* b, int64_t ldb, int b_fmt, const uint8_t* b_scales,
            void* c, int64_t ldc, int c_dtype, void* stream);

/*
 * gaussws_sample -- GaussWS sampled weight [GWS "What carries the argument"]:
 *
 *   w_hat[r][c] = bf16( fp32( w[r][c] + R(r, c) * ldexp(amax_bl, 1 - b_bl) ) )
 *
 * over 32x32 blocks bl (partial at the edges), amax_bl = max |w| in the
 * block, b_bl = bitwidths[r / 32][c / 32] (int8, read as an integer
 * exponent), R the nearest integer to N(0,1)/2 with support folded to
 * {-2..2}: |R| = 0, 1, 2 as |Z| < 1, 1 <= |Z| < 3, |Z| >= 3 (P(R = 0) =
 * 0.6827).  The page's bitwise approximation of R is not printed; R is drawn
 * here by its definition from 32 uniform bits per element: bit 31 the sign,
 * bits 0..30 against round(erf(1/sqrt 2) * 2^31) and round(erf(3/sqrt 2) *
 * 2^31).  The bits are the counter-based Philox4x64-10 (Salmon et al.,
 * SC'11) with key (seed, stream_id) and counter (c / 8, r, 0, 0): output
 * word (c % 8) / 2, low half for even c, high half for odd c.  The result
 * depends only on (seed, stream_id, r, c) and the inputs, so it is
 * deterministic and reproducible across calls and launch shapes.
 *   w:         [rows][ldw >= cols] fp32 or bf16 (w_dtype).
 *   bitwidths: [ceil(rows / 32)][ceil(cols / 32)] int8.
 *   w_hat:     [rows][ldo >= cols] bf16 bit patterns, overwritten.
 * Requires cols % 8 == 0.  The fp32 sum is rounded to bf16 to nearest even.
 */
int gaussws_sample(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ldw,
                   const int8_t* bitwidths, uint64_t seed, uint64_t stream_id, uint16_t* w_hat,
                   int64_t ldo, void* stream);

/* Static description of a status code (never NULL). */
const char* mxfp8_status_string(int status);

/* MXFP8_VERSION of the built library. */
int mxfp8_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MXFP8_H */
