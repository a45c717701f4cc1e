/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for hybrid-granularity
 * FP8 quantization with power-of-two (E8M0) scales and the block-scaled FP8
 * GEMM that consumes it.
 *
 * TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark are its only users.  The product library
 * never includes, links or calls it, and it includes nothing from the
 * product.  Built with gcc -O2, no fast-math, no intrinsics.  All arithmetic
 * is fp64; every quantity that the definitions fix exactly is computed
 * exactly (power-of-two scaling of an fp32/bf16 value is exact in fp64).
 *
 * Sources (web pages; titles as printed on them):
 *   [FP8F] "FP8 Formats for Deep Learning" -- review page, "The pith",
 *          "Core claim" and the quoted abstract: E4M3 (4 exponent bits,
 *          3 mantissa bits) has no infinities and a single NaN mantissa
 *          pattern; E5M2 (5/2 bits) follows IEEE 754 for special values.
 *          "Axiom & Free-Parameter Ledger": the standard floating-point
 *          representation and rounding rules hold apart from E4M3's specials.
 *   [INFR] "A Comprehensive FP8 Training Recipe for Reasoning-Enhanced
 *          Language Models" -- review page, "Core claim" and "What carries
 *          the argument": weights quantized per block, activations per token,
 *          scaling factors stored as UE8M0 (exponent only) and rounded UP to a
 *          power of two so that the quantized tensor stays inside the FP8
 *          range; Figures 1 and 2 (per-block / per-token granularity).
 *          "Axiom & Free-Parameter Ledger": the weight block size is not
 *          reported by the paper.
 *   [MXTI] "Characterization and Mitigation of Training Instabilities in
 *          Microscaling Formats" -- review page, "What carries the argument":
 *          MX blocks share one power-of-two scale; for MXFP8 E4M3 a scaled
 *          value above 0.875 of the block's binade top is clamped to the
 *          largest code; Fig. 5 caption: E4M3 successive-code gaps, clamping
 *          once the scaled magnitude exceeds the representable limit.
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes of the repository):
 *   R1  group sizes: 1x128 along the contiguous axis for tokens, 128x128 for
 *       weight tiles, 32 along rows for MX (the pages give no sizes).
 *   R2  E4M3/E5M2 exponent bias = 2^(ebits-1)-1 (IEEE style, "standard
 *       rules"); with E4M3's single NaN pattern S.1111.111 this makes its
 *       largest finite value 448.
 *   R3  the cast is round-to-nearest, ties-to-even, and saturates finite
 *       overflow to the largest finite code; the sign of zero is kept.
 *   R4  round-up scale: e = smallest integer with amax <= fmax * 2^e,
 *       stored as the E8M0 byte e + 127, e clamped to [-127, 127];
 *       amax == 0 gives e = -127 (byte 0).
 *   R5  MX scale: X = floor(log2 amax) - emax_elem, where emax_elem is the
 *       binade exponent of the format's largest finite value (8 for E4M3,
 *       15 for E5M2), clamped to [-127, 127]; amax == 0 gives -127.
 *   R6  a group that runs past the end of its axis is partial; its amax is
 *       taken over the elements present.
 *   R7  the GEMM result is the exact sum over k of the dequantized products;
 *       here it is accumulated in fp64 (sequential over k), together with
 *       sum_k |a*b| which sizes the tolerance.
 *   R8  "FP8 with an FP32 scale" (named on the recipe page's review as a
 *       variant of its Table 4, not defined there): the scale is not rounded
 *       to a power of two but is the fp32 quotient s = amax / fmax (IEEE
 *       single precision, round to nearest even; s = 1 when that quotient
 *       is zero, i.e. amax == 0 or amax < fmax * 2^-150), and each code is
 *       the saturating cast of the fp32 quotient x / s.  Both
 *       divisions are IEEE fp32 operations, so the codes are fixed bits.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* Format description [FP8F]                                              */
/* ---------------------------------------------------------------------- */

static int mant_bits(int fmt) { return fmt == 0 ? 3 : 2; }
static int exp_bits(int fmt) { return fmt == 0 ? 4 : 5; }
static int exp_bias(int fmt) { return (1 << (exp_bits(fmt) - 1)) - 1; } /* R2 */

/* Decode one FP8 code to its real value [FP8F]. */
double orc_decode(int fmt, uint8_t code) {
  const int mb = mant_bits(fmt), eb = exp_bits(fmt), bias = exp_bias(fmt);
  const int s = code >> 7;
  const int E = (code >> mb) & ((1 << eb) - 1);
  const int m = code & ((1 << mb) - 1);
  const double sign = s ? -1.0 : 1.0;
  const int Emax = (1 << eb) - 1;
  if (fmt == 0) {
    /* E4M3: no infinities; the one NaN pattern is all-ones exponent and
     * all-ones mantissa. Every other all-ones-exponent code is a number. */
    if (E == Emax && m == (1 << mb) - 1) return NAN;
  } else {
    /* E5M2: IEEE 754 specials -- all-ones exponent is inf (m == 0) or NaN. */
    if (E == Emax) return m == 0 ? sign * INFINITY : NAN;
  }
  if (E == 0) /* subnormal: 0.m * 2^(1-bias) */
    return sign * ldexp((double)m, 1 - bias - mb);
  return sign * ldexp((double)((1 << mb) + m), E - bias - mb); /* 1.m * 2^(E-bias) */
}

/* Largest finite value of each format: the maximum over all 256 decoded
 * codes, tabulated once when the library is loaded. */
static double g_fmax[2];
__attribute__((constructor)) static void init_fmax(void) {
  for (int fmt = 0; fmt < 2; ++fmt) {
    double best = 0.0;
    for (int c = 0; c < 256; ++c) {
      double v = orc_decode(fmt, (uint8_t)c);
      if (isfinite(v) && v > best) best = v;
    }
    g_fmax[fmt] = best;
  }
}
static double fmax_of(int fmt) { return g_fmax[fmt]; }

/* floor(log2 a) for finite a > 0: the integer p with 2^p <= a < 2^(p+1).
 * frexp returns a = f * 2^q with f in [0.5, 1), so p = q - 1. */
static int floor_log2(double a) {
  int q;
  frexp(a, &q);
  return q - 1;
}

/* Saturating round-to-nearest-even cast of a real value to FP8 (R3).
 * Non-finite inputs: NaN -> the NaN code 0x7F with x's sign bit; +-inf ->
 * +-fmax in E4M3 (no infinities, saturating) and +-inf in E5M2. */
uint8_t orc_encode(int fmt, double x) {
  const int mb = mant_bits(fmt), bias = exp_bias(fmt);
  const int emin = 1 - bias; /* exponent of the smallest normal binade */
  const double fmax = fmax_of(fmt);
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  double a = fabs(x);
  if (isinf(a)) {
    if (fmt == 0) return (uint8_t)(sign | orc_encode(fmt, fmax));
    return (uint8_t)(sign | 0x7C);
  }
  /* binade of a, but never below the subnormal binade */
  int e = a == 0.0 ? emin : floor_log2(a);
  if (e < emin) e = emin;
  /* quantum (spacing of representable values) in that binade */
  const double quantum = ldexp(1.0, e - mb);
  const double r = nearbyint(a / quantum); /* exact quotient; ties to even (default mode) */
  double v = r * quantum;
  if (v > fmax) v = fmax; /* saturate */
  if (v == 0.0) return sign;
  /* write v back as fields; r may have carried into the next binade */
  int ev = floor_log2(v);
  if (ev < emin) { /* subnormal: E = 0, v = m * 2^(emin - mb) */
    int m = (int)(v / ldexp(1.0, emin - mb));
    return (uint8_t)(sign | m);
  }
  int m = (int)((v / ldexp(1.0, ev) - 1.0) * (double)(1 << mb));
  return (uint8_t)(sign | ((ev + bias) << mb) | m);
}

/* Round-up power-of-two scale exponent, R4 [INFR "What carries the argument"]:
 * the smallest integer e with amax <= fmax * 2^e, by direct search. */
int orc_scale_exp_ceil(int fmt, double amax) {
  const double fmax = fmax_of(fmt);
  for (int e = -127; e <= 127; ++e)
    if (amax <= ldexp(fmax, e)) return e;
  return 127; /* not reached for finite fp32 inputs (fp32 max < 448 * 2^127) */
}

/* OCP MX shared exponent, R5 [MXTI "What carries the argument"]. */
int orc_scale_exp_floor(int fmt, double amax) {
  if (amax == 0.0) return -127;
  const int emax_elem = floor_log2(fmax_of(fmt));
  int X = floor_log2(amax) - emax_elem;
  if (X < -127) X = -127;
  if (X > 127) X = 127;
  return X;
}

/* ---------------------------------------------------------------------- */
/* Element access                                                          */
/* ---------------------------------------------------------------------- */

/* Widen one input element to fp64 exactly (dtype 0 = fp32, 1 = bf16 bits). */
static double load_elem(const void* base, int dtype, int64_t idx) {
  if (dtype == 0) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

/* ---------------------------------------------------------------------- */
/* Quantizers [INFR, MXTI]                                                 */
/* ---------------------------------------------------------------------- */

/* Token-wise 1x128 groups along each row (activations, gradients) [INFR,
 * "What carries the argument", Fig. 2]: per (row r, group g) the amax, the
 * round-up scale, then the cast of every element of the group.
 * q[r*ldq + c], s[r*ceil(cols/128) + g] = e + 127. */
void orc_quantize_rows(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                       int fmt, uint8_t* q, int64_t ldq, uint8_t* s) {
  const int64_t G = 128, ng = ceil_div(cols, G);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < ng; ++g) {
      const int64_t c0 = g * G, c1 = min64(c0 + G, cols);
      double amax = 0.0;
      for (int64_t c = c0; c < c1; ++c) {
        double a = fabs(load_elem(x, dtype, r * ldx + c));
        if (a > amax) amax = a;
      }
      const int e = orc_scale_exp_ceil(fmt, amax);
      s[r * ng + g] = (uint8_t)(e + 127);
      for (int64_t c = c0; c < c1; ++c)
        q[r * ldq + c] = orc_encode(fmt, ldexp(load_elem(x, dtype, r * ldx + c), -e));
    }
}

/* Token-wise groups taken along the token axis and written transposed, for
 * the weight-gradient contraction over tokens: x is [rows = tokens][cols =
 * channels]; for each channel c and group t of 128 consecutive tokens:
 * qt[c*ldq + r], st[c*ceil(rows/128) + t] = e + 127. */
void orc_quantize_cols_t(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                         int fmt, uint8_t* qt, int64_t ldq, uint8_t* st) {
  const int64_t G = 128, ng = ceil_div(rows, G);
  for (int64_t c = 0; c < cols; ++c)
    for (int64_t t = 0; t < ng; ++t) {
      const int64_t r0 = t * G, r1 = min64(r0 + G, rows);
      double amax = 0.0;
      for (int64_t r = r0; r < r1; ++r) {
        double a = fabs(load_elem(x, dtype, r * ldx + c));
        if (a > amax) amax = a;
      }
      const int e = orc_scale_exp_ceil(fmt, amax);
      st[c * ng + t] = (uint8_t)(e + 127);
      for (int64_t r = r0; r < r1; ++r)
        qt[c * ldq + r] = orc_encode(fmt, ldexp(load_elem(x, dtype, r * ldx + c), -e));
    }
}

/* Block-wise 128x128 tiles (weights) [INFR "What carries the argument",
 * Fig. 1]: one round-up scale per tile; q keeps w's layout;
 * s[i*ceil(cols/128) + j] = e + 127. */
void orc_quantize_block(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw,
                        int fmt, uint8_t* q, int64_t ldq, uint8_t* s) {
  const int64_t G = 128, nbr = ceil_div(rows, G), nbc = ceil_div(cols, G);
  for (int64_t i = 0; i < nbr; ++i)
    for (int64_t j = 0; j < nbc; ++j) {
      const int64_t r0 = i * G, r1 = min64(r0 + G, rows);
      const int64_t c0 = j * G, c1 = min64(c0 + G, cols);
      double amax = 0.0;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          double a = fabs(load_elem(w, dtype, r * ldw + c));
          if (a > amax) amax = a;
        }
      const int e = orc_scale_exp_ceil(fmt, amax);
      s[i * nbc + j] = (uint8_t)(e + 127);
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c)
          q[r * ldq + c] = orc_encode(fmt, ldexp(load_elem(w, dtype, r * ldw + c), -e));
    }
}

/* MX quantization, 32-element blocks along each row sharing one E8M0 scale
 * [MXTI "What carries the argument", Fig. 5]: rule 1 = OCP floor rule (R5),
 * whose scaled values can exceed fmax and then saturate; rule 0 = the
 * round-up rule (R4).  counts (nullable) receives, per block, the number of
 * elements whose scaled magnitude exceeds fmax -- the clamped fraction that
 * the instability page proposes to monitor ("Reading between the lines").
 * s and counts are [rows][ceil(cols/32)]. */
void orc_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                     int fmt, int rule, uint8_t* q, int64_t ldq, uint8_t* s, uint8_t* counts) {
  const int64_t G = 32, ng = ceil_div(cols, G);
  const double fmax = fmax_of(fmt);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < ng; ++g) {
      const int64_t c0 = g * G, c1 = min64(c0 + G, cols);
      double amax = 0.0;
      for (int64_t c = c0; c < c1; ++c) {
        double a = fabs(load_elem(x, dtype, r * ldx + c));
        if (a > amax) amax = a;
      }
      const int e = rule == 1 ? orc_scale_exp_floor(fmt, amax) : orc_scale_exp_ceil(fmt, amax);
      s[r * ng + g] = (uint8_t)(e + 127);
      int clamped = 0;
      for (int64_t c = c0; c < c1; ++c) {
        const double v = ldexp(load_elem(x, dtype, r * ldx + c), -e);
        if (fabs(v) > fmax) ++clamped;
        q[r * ldq + c] = orc_encode(fmt, v);
      }
      if (counts) counts[r * ng + g] = (uint8_t)clamped;
    }
}

/* ---------------------------------------------------------------------- */
/* Quantizers with fp32 scales (R8)                                         */
/* ---------------------------------------------------------------------- */

/* The fp32 scale of a group whose largest magnitude is amax (an fp32 value:
 * the inputs are fp32 or bf16): amax / fmax in IEEE single precision; a
 * quotient that rounds to zero (amax == 0, or amax below fmax * 2^-150) is
 * replaced by 1, so that every quotient x / s below is finite. */
float orc_scale_f32(int fmt, float amax) {
  const float fmax = (float)fmax_of(fmt);
  const float s = amax / fmax;
  return s == 0.0f ? 1.0f : s;
}

/* Code of one element under an fp32 scale: the fp32 quotient x / s, then
 * the saturating cast (R3). */
static uint8_t encode_div(int fmt, double x, float s) {
  const float v = (float)x / s; /* x is an fp32 (or bf16) value: exact */
  return orc_encode(fmt, (double)v);
}

/* Largest magnitude of the elements r0..r1-1 x c0..c1-1, as fp32. */
static float group_amax(const void* x, int dtype, int64_t ldx, int64_t r0, int64_t r1, int64_t c0,
                        int64_t c1) {
  double amax = 0.0;
  for (int64_t r = r0; r < r1; ++r)
    for (int64_t c = c0; c < c1; ++c) {
      const double a = fabs(load_elem(x, dtype, r * ldx + c));
      if (a > amax) amax = a;
    }
  return (float)amax; /* exact: amax is one of the fp32 inputs */
}

/* Token-wise 1x128 groups along rows with fp32 scales (R8);
 * s[r*ceil(cols/128) + g] = the group's fp32 scale. */
void orc_quantize_rows_f32s(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                            int fmt, uint8_t* q, int64_t ldq, float* s) {
  const int64_t G = 128, ng = ceil_div(cols, G);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < ng; ++g) {
      const int64_t c0 = g * G, c1 = min64(c0 + G, cols);
      const float sc = orc_scale_f32(fmt, group_amax(x, dtype, ldx, r, r + 1, c0, c1));
      s[r * ng + g] = sc;
      for (int64_t c = c0; c < c1; ++c) q[r * ldq + c] = encode_div(fmt, load_elem(x, dtype, r * ldx + c), sc);
    }
}

/* 128-token groups down columns, written transposed, with fp32 scales (R8):
 * qt[c*ldq + r], st[c*ceil(rows/128) + t]. */
void orc_quantize_cols_t_f32s(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                              int fmt, uint8_t* qt, int64_t ldq, float* st) {
  const int64_t G = 128, ng = ceil_div(rows, G);
  for (int64_t c = 0; c < cols; ++c)
    for (int64_t t = 0; t < ng; ++t) {
      const int64_t r0 = t * G, r1 = min64(r0 + G, rows);
      const float sc = orc_scale_f32(fmt, group_amax(x, dtype, ldx, r0, r1, c, c + 1));
      st[c * ng + t] = sc;
      for (int64_t r = r0; r < r1; ++r) qt[c * ldq + r] = encode_div(fmt, load_elem(x, dtype, r * ldx + c), sc);
    }
}

/* 128x128 tiles with fp32 scales (R8): s[i*ceil(cols/128) + j]. */
void orc_quantize_block_f32s(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw,
                             int fmt, uint8_t* q, int64_t ldq, float* s) {
  const int64_t G = 128, nbr = ceil_div(rows, G), nbc = ceil_div(cols, G);
  for (int64_t i = 0; i < nbr; ++i)
    for (int64_t j = 0; j < nbc; ++j) {
      const int64_t r0 = i * G, r1 = min64(r0 + G, rows);
      const int64_t c0 = j * G, c1 = min64(c0 + G, cols);
      const float sc = orc_scale_f32(fmt, group_amax(w, dtype, ldw, r0, r1, c0, c1));
      s[i * nbc + j] = sc;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) q[r * ldq + c] = encode_div(fmt, load_elem(w, dtype, r * ldw + c), sc);
    }
}

/* ---------------------------------------------------------------------- */
/* GaussWS fake quantization (R9)                                          */
/* ---------------------------------------------------------------------- */

/* Philox4x64-10: ten rounds of two 64x64 -> 128-bit products with the
 * published multipliers, the key bumped by the published Weyl increments
 * after each round. */
void orc_philox4x64(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    const unsigned __int128 p0 = (unsigned __int128)M0 * x0, p1 = (unsigned __int128)M1 * x2;
    const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
    const uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* R from 32 uniform bits (R9): thresholds on the low 31 bits at
 * P(|Z| < 1) = erf(1/sqrt 2) and P(|Z| < 3) = erf(3/sqrt 2) of a standard
 * normal Z, times 2^31 and rounded to the nearest integer (computed once
 * when the library is loaded). */
static uint32_t g_r_t0, g_r_t1;
__attribute__((constructor)) static void init_gaussws_thresholds(void) {
  const double two31 = 2147483648.0;
  g_r_t0 = (uint32_t)floor(erf(1.0 / sqrt(2.0)) * two31 + 0.5);
  g_r_t1 = (uint32_t)floor(erf(3.0 / sqrt(2.0)) * two31 + 0.5);
}

int orc_gaussws_r(uint32_t u) {
  const uint32_t m = u & 0x7FFFFFFFu;
  const int mag = m < g_r_t0 ? 0 : (m < g_r_t1 ? 1 : 2);
  return (u >> 31) ? -mag : mag;
}

/* The 32 uniform bits of element (r, c). */
static uint32_t gaussws_bits(uint64_t seed, uint64_t stream, int64_t r, int64_t c) {
  const uint64_t ctr[4] = {(uint64_t)(c / 8), (uint64_t)r, 0, 0};
  const uint64_t key[2] = {seed, stream};
  uint64_t out[4];
  orc_philox4x64(ctr, key, out);
  const uint64_t w = out[(c % 8) / 2];
  return (c % 2) ? (uint32_t)(w >> 32) : (uint32_t)w;
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept NaN). */
static uint16_t bf16_rne_bits(float f) {
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40);
  const uint32_t lsb = (b >> 16) & 1u;
  return (uint16_t)((b + 0x7FFFu + lsb) >> 16);
}

/* R for every element of a [rows][cols] tensor (int8, for the tests). */
void orc_gaussws_noise(uint64_t seed, uint64_t stream, int64_t rows, int64_t cols, int8_t* r_out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) r_out[r * cols + c] = (int8_t)orc_gaussws_r(gaussws_bits(seed, stream, r, c));
}

/* w_hat[r][c] (bf16 bits) = bf16(fp32(w + R * ldexp(max_bl |w|, 1 - b_t))),
 * blocks of 32x32 (partial at the edges), b_t[ceil(rows/32)][ceil(cols/32)];
 * for the block rows [i0, i1) (rows keep their index in the whole tensor). */
void orc_gaussws(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw, const int8_t* bt,
                 uint64_t seed, uint64_t stream, uint16_t* out, int64_t ldo, int64_t i0, int64_t i1) {
  const int64_t G = 32, nbc = ceil_div(cols, G);
  for (int64_t i = i0; i < i1; ++i)
    for (int64_t j = 0; j < nbc; ++j) {
      const int64_t r0 = i * G, r1 = min64(r0 + G, rows);
      const int64_t c0 = j * G, c1 = min64(c0 + G, cols);
      double amax = 0.0;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          const double a = fabs(load_elem(w, dtype, r * ldw + c));
          if (a > amax) amax = a;
        }
      const float scale = ldexpf((float)amax, 1 - (int)bt[i * nbc + j]);
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          const float noise = (float)orc_gaussws_r(gaussws_bits(seed, stream, r, c)) * scale;
          const float v = (float)load_elem(w, dtype, r * ldw + c) + noise;
          out[r * ldo + c] = bf16_rne_bits(v);
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Block-scaled GEMM [INFR "What carries the argument"; R7]                */
/* ---------------------------------------------------------------------- */

/* Dequantized A element: dec(code) * 2^(scale byte - 127), one scale per
 * (row m, 128-wide K block). */
static double a_value(int64_t K, const uint8_t* a, int64_t lda, int a_fmt, const uint8_t* sa,
                      int64_t m, int64_t k) {
  const int64_t nkb = ceil_div(K, 128);
  return ldexp(orc_decode(a_fmt, a[m * lda + k]), (int)sa[m * nkb + k / 128] - 127);
}

/* Dequantized B element at logical (k, n).  Storage: layout 0 = [N][K],
 * layout 1 = [K][N].  Scales: mode 0 = one per 128x128 tile of the storage
 * ([N/128][K/128] or [K/128][N/128]); mode 1 = one per (n, 128-wide K block),
 * [N][K/128]. */
static double b_value(int64_t N, int64_t K, const uint8_t* b, int64_t ldb, int b_fmt,
                      int b_layout, const uint8_t* sb, int b_scale, int64_t k, int64_t n) {
  const int64_t nkb = ceil_div(K, 128), nnb = ceil_div(N, 128);
  const uint8_t code = b_layout == 0 ? b[n * ldb + k] : b[k * ldb + n];
  int byte;
  if (b_scale == 1) byte = sb[n * nkb + k / 128];
  else if (b_layout == 0) byte = sb[(n / 128) * nkb + k / 128];
  else byte = sb[(k / 128) * nnb + n / 128];
  return ldexp(orc_decode(b_fmt, code), byte - 127);
}

/* y[m][n] = sum_k a(m,k) * b(k,n) and t[m][n] = sum_k |a(m,k) * b(k,n)| for
 * rows m in [m0, m1), all n; y and t are indexed [m*ldy + n].  B is
 * dequantized once into an fp64 [N][K] array, each row of A into [K]. */
void orc_gemm(int64_t M, int64_t N, int64_t K,
              const uint8_t* a, int64_t lda, int a_fmt, const uint8_t* sa,
              const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
              const uint8_t* sb, int b_scale,
              int64_t m0, int64_t m1, double* y, double* t, int64_t ldy) {
  (void)M;
  double* bd = (double*)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
  double* ad = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
  if (!bd || !ad) { free(bd); free(ad); abort(); }
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k)
      bd[n * K + k] = b_value(N, K, b, ldb, b_fmt, b_layout, sb, b_scale, k, n);
  for (int64_t m = m0; m < m1; ++m) {
    for (int64_t k = 0; k < K; ++k) ad[k] = a_value(K, a, lda, a_fmt, sa, m, k);
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0, mag = 0.0;
      const double* bn = bd + n * K;
      for (int64_t k = 0; k < K; ++k) {
        const double p = ad[k] * bn[k];
        acc += p;
        mag += fabs(p);
      }
      y[m * ldy + n] = acc;
      t[m * ldy + n] = mag;
    }
  }
  free(ad);
  free(bd);
}

/* The same sums for an explicit list of output elements (ii[i], jj[i]),
 * computed one by one; for spot checks at sizes where the full product is
 * too slow on a CPU. */
void orc_gemm_elems(int64_t M, int64_t N, int64_t K,
                    const uint8_t* a, int64_t lda, int a_fmt, const uint8_t* sa,
                    const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
                    const uint8_t* sb, int b_scale,
                    const int64_t* ii, const int64_t* jj, int64_t n, double* y, double* t) {
  (void)M;
  for (int64_t i = 0; i < n; ++i) {
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double p = a_value(K, a, lda, a_fmt, sa, ii[i], k) *
                       b_value(N, K, b, ldb, b_fmt, b_layout, sb, b_scale, k, jj[i]);
      acc += p;
      mag += fabs(p);
    }
    y[i] = acc;
    t[i] = mag;
  }
}

/* GEMM over operands with fp32 scales (R8, R7): a(m,k) = dec(A[m][k]) *
 * sa[m][k/128], b(k,n) = dec(B(k,n)) * sb(k/128, n) with the scale layouts of
 * orc_gemm (floats instead of bytes).  Each dequantized element is exact in
 * fp64 (a 4-bit significand times a 24-bit one). */
static double a_value_f32s(int64_t K, const uint8_t* a, int64_t lda, int a_fmt, const float* sa, int64_t m,
                           int64_t k) {
  const int64_t nkb = ceil_div(K, 128);
  return orc_decode(a_fmt, a[m * lda + k]) * (double)sa[m * nkb + k / 128];
}

static double b_value_f32s(int64_t N, int64_t K, const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
                           const float* sb, int b_scale, int64_t k, int64_t n) {
  const int64_t nkb = ceil_div(K, 128), nnb = ceil_div(N, 128);
  const uint8_t code = b_layout == 0 ? b[n * ldb + k] : b[k * ldb + n];
  double scale;
  if (b_scale == 1) scale = sb[n * nkb + k / 128];
  else if (b_layout == 0) scale = sb[(n / 128) * nkb + k / 128];
  else scale = sb[(k / 128) * nnb + n / 128];
  return orc_decode(b_fmt, code) * scale;
}

void orc_gemm_f32s(int64_t M, int64_t N, int64_t K,
                   const uint8_t* a, int64_t lda, int a_fmt, const float* sa,
                   const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
                   const float* sb, int b_scale,
                   int64_t m0, int64_t m1, double* y, double* t, int64_t ldy) {
  (void)M;
  double* bd = (double*)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
  double* ad = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
  if (!bd || !ad) { free(bd); free(ad); abort(); }
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k)
      bd[n * K + k] = b_value_f32s(N, K, b, ldb, b_fmt, b_layout, sb, b_scale, k, n);
  for (int64_t m = m0; m < m1; ++m) {
    for (int64_t k = 0; k < K; ++k) ad[k] = a_value_f32s(K, a, lda, a_fmt, sa, m, k);
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0, mag = 0.0;
      const double* bn = bd + n * K;
      for (int64_t k = 0; k < K; ++k) {
        const double p = ad[k] * bn[k];
        acc += p;
        mag += fabs(p);
      }
      y[m * ldy + n] = acc;
      t[m * ldy + n] = mag;
    }
  }
  free(ad);
  free(bd);
}

void orc_gemm_f32s_elems(int64_t M, int64_t N, int64_t K,
                         const uint8_t* a, int64_t lda, int a_fmt, const float* sa,
                         const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
                         const float* sb, int b_scale,
                         const int64_t* ii, const int64_t* jj, int64_t n, double* y, double* t) {
  (void)M;
  for (int64_t i = 0; i < n; ++i) {
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double p = a_value_f32s(K, a, lda, a_fmt, sa, ii[i], k) *
                       b_value_f32s(N, K, b, ldb, b_fmt, b_layout, sb, b_scale, k, jj[i]);
      acc += p;
      mag += fabs(p);
    }
    y[i] = acc;
    t[i] = mag;
  }
}

/* MX GEMM ["Characterization and Mitigation of Training Instabilities in
 * Microscaling Formats", "What carries the argument": a block of 32
 * consecutive elements shares one E8M0 scale, the element's value being the
 * scale times the decoded FP8 element; the GEMM runs on such operands].
 * Both operands are blocked along K: A [M][K] with scales [M][K/32], B stored
 * [N][K] with scales [N][K/32] (what the MX quantizer produces along rows).
 * y and t as in orc_gemm, for rows [m0, m1). */
static double mx_value(int64_t K, const uint8_t* x, int64_t ldx, int fmt, const uint8_t* s,
                       int64_t r, int64_t k) {
  const int64_t nkc = ceil_div(K, 32);
  return ldexp(orc_decode(fmt, x[r * ldx + k]), (int)s[r * nkc + k / 32] - 127);
}

void orc_mx_gemm(int64_t M, int64_t N, int64_t K,
                 const uint8_t* a, int64_t lda, int a_fmt, const uint8_t* sa,
                 const uint8_t* b, int64_t ldb, int b_fmt, const uint8_t* sb,
                 int64_t m0, int64_t m1, double* y, double* t, int64_t ldy) {
  (void)M;
  double* bd = (double*)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
  double* ad = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
  if (!bd || !ad) { free(bd); free(ad); abort(); }
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) bd[n * K + k] = mx_value(K, b, ldb, b_fmt, sb, n, k);
  for (int64_t m = m0; m < m1; ++m) {
    for (int64_t k = 0; k < K; ++k) ad[k] = mx_value(K, a, lda, a_fmt, sa, m, k);
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0, mag = 0.0;
      const double* bn = bd + n * K;
      for (int64_t k = 0; k < K; ++k) {
        const double p = ad[k] * bn[k];
        acc += p;
        mag += fabs(p);
      }
      y[m * ldy + n] = acc;
      t[m * ldy + n] = mag;
    }
  }
  free(ad);
  free(bd);
}

void orc_mx_gemm_elems(int64_t M, int64_t N, int64_t K,
                       const uint8_t* a, int64_t lda, int a_fmt, const uint8_t* sa,
                       const uint8_t* b, int64_t ldb, int b_fmt, const uint8_t* sb,
                       const int64_t* ii, const int64_t* jj, int64_t n, double* y, double* t) {
  (void)M;
  (void)N;
  for (int64_t i = 0; i < n; ++i) {
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double p = mx_value(K, a, lda, a_fmt, sa, ii[i], k) * mx_value(K, b, ldb, b_fmt, sb, jj[i], k);
      acc += p;
      mag += fabs(p);
    }
    y[i] = acc;
    t[i] = mag;
  }
}

/* ---------------------------------------------------------------------- */
/* Array helpers for the tests (loops over the scalar functions above)      */
/* ---------------------------------------------------------------------- */

void orc_decode_array(int fmt, const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_decode(fmt, codes[i]);
}

void orc_encode_array(int fmt, const double* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_encode(fmt, x[i]);
}

/* Encode the fp32 values whose bit patterns are start, start+1, ...,
 * start+n-1 (an exhaustive sweep over fp32 is a sequence of such calls). */
void orc_encode_f32_range(int fmt, uint32_t start, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t bits = start + (uint32_t)i;
    float f;
    memcpy(&f, &bits, sizeof f);
    out[i] = orc_encode(fmt, (double)f);
  }
}
