/* Host driver for the CPU oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every function runs on exactly-sized heap
 * buffers (so any access past a tensor is reported), on ragged shapes, both
 * formats, both input dtypes, both scale rules and every GEMM layout, plus a
 * few invariants that need no second implementation (code round trips, the
 * round-up rule never saturating, sum|a*b| >= |sum a*b|). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static int fails = 0;
#define CHECK(c)                                                    \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #c); \
      ++fails;                                                      \
    }                                                               \
  } while (0)

static uint64_t rng = 88172645463325252ull;
static uint32_t next32(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (uint32_t)(rng >> 11);
}
static double unif(void) { return (next32() + 0.5) / 4294967296.0; }
static double gauss(void) { return sqrt(-2.0 * log(unif())) * cos(6.283185307179586 * unif()); }

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

/* rows x cols input (row pitch ld) of fp32 or bf16 patterns, N(0,1) times 2^k. */
static void* make_input(int dtype, int64_t rows, int64_t cols, int64_t ld, int k) {
  const size_t es = dtype ? 2 : 4;
  unsigned char* x = xmalloc((size_t)(rows * ld) * es);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < ld; ++c) {
      float v = (float)ldexp(gauss(), k);
      if (c % 37 == 5) v = 0.0f;
      uint32_t b;
      memcpy(&b, &v, 4);
      if (dtype) {
        uint16_t h = (uint16_t)(b >> 16);
        memcpy(x + (size_t)(r * ld + c) * 2, &h, 2);
      } else {
        memcpy(x + (size_t)(r * ld + c) * 4, &b, 4);
      }
    }
  return x;
}

static void codec(void) {
  for (int fmt = 0; fmt < 2; ++fmt)
    for (int c = 0; c < 256; ++c) {
      const double v = orc_decode(fmt, (uint8_t)c);
      if (isfinite(v)) CHECK(orc_decode(fmt, orc_encode(fmt, v)) == v);
    }
  uint8_t* out = xmalloc(1 << 16);
  orc_encode_f32_range(0, 0x3F000000u, 1 << 16, out);
  orc_encode_f32_range(1, 0xFFFF0000u, 1 << 16, out);
  free(out);
  double vals[5] = {0.0, -0.0, 1e-30, 448.0 * 1.0001, -70000.0};
  uint8_t codes[5];
  orc_encode_array(0, vals, 5, codes);
  CHECK(codes[3] == 0x7E && codes[4] == 0xFE);
  double back[5];
  orc_decode_array(1, codes, 5, back);
  for (int e = -140; e < 140; e += 7) {
    CHECK(orc_scale_exp_ceil(0, ldexp(1.3, e)) >= -127);
    CHECK(orc_scale_exp_floor(1, ldexp(1.3, e)) <= 127);
  }
}

static void quantizers(void) {
  const int64_t shapes[3][2] = {{7, 48}, {130, 272}, {33, 144}};
  for (int si = 0; si < 3; ++si)
    for (int dtype = 0; dtype < 2; ++dtype)
      for (int fmt = 0; fmt < 2; ++fmt) {
        const int64_t rows = shapes[si][0], cols = shapes[si][1], ld = cols + 16;
        void* x = make_input(dtype, rows, cols, ld, si * 5 - 3);
        const int64_t ng = (cols + 127) / 128, ngt = (rows + 127) / 128;
        uint8_t* q = xmalloc((size_t)(rows * cols));
        uint8_t* s = xmalloc((size_t)(rows * ng));
        orc_quantize_rows(x, dtype, rows, cols, ld, fmt, q, cols, s);
        for (int64_t i = 0; i < rows * ng; ++i) CHECK(s[i] <= 254);
        uint8_t* qt = xmalloc((size_t)(cols * rows));
        uint8_t* stt = xmalloc((size_t)(cols * ngt));
        orc_quantize_cols_t(x, dtype, rows, cols, ld, fmt, qt, rows, stt);
        uint8_t* sb = xmalloc((size_t)(ngt * ng));
        orc_quantize_block(x, dtype, rows, cols, ld, fmt, q, cols, sb);
        for (int64_t i = 0; i < rows * cols; ++i) CHECK((q[i] & 0x7F) <= (fmt ? 0x7B : 0x7E));
        float* sf = xmalloc(sizeof(float) * (size_t)(rows * ng));
        orc_quantize_rows_f32s(x, dtype, rows, cols, ld, fmt, q, cols, sf);
        float* sft = xmalloc(sizeof(float) * (size_t)(cols * ngt));
        orc_quantize_cols_t_f32s(x, dtype, rows, cols, ld, fmt, qt, rows, sft);
        float* sfb = xmalloc(sizeof(float) * (size_t)(ngt * ng));
        orc_quantize_block_f32s(x, dtype, rows, cols, ld, fmt, q, cols, sfb);
        for (int rule = 0; rule < 2; ++rule) {
          const int64_t nb = (cols + 31) / 32;
          uint8_t* ms = xmalloc((size_t)(rows * nb));
          uint8_t* mc = xmalloc((size_t)(rows * nb));
          orc_mx_quantize(x, dtype, rows, cols, ld, fmt, rule, q, cols, ms, mc);
          for (int64_t i = 0; i < rows * nb; ++i) CHECK(mc[i] <= 32 && (rule == 1 || mc[i] == 0));
          free(ms);
          free(mc);
        }
        free(x); free(q); free(s); free(qt); free(stt); free(sb); free(sf); free(sft); free(sfb);
      }
}

static uint8_t rand_code(int fmt) {
  for (;;) {
    const uint8_t c = (uint8_t)next32();
    if (isfinite(orc_decode(fmt, c))) return c;
  }
}

static void gemms(void) {
  const int64_t M = 37, N = 133, K = 384, nkb = K / 128, nnb = (N + 127) / 128;
  uint8_t* a = xmalloc((size_t)(M * K));
  uint8_t* bnk = xmalloc((size_t)(N * K));
  uint8_t* bkn = xmalloc((size_t)(K * N));
  for (int64_t i = 0; i < M * K; ++i) a[i] = rand_code(0);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) bkn[k * N + n] = bnk[n * K + k] = rand_code(1);
  uint8_t* sa = xmalloc((size_t)(M * nkb));
  uint8_t* sbr = xmalloc((size_t)(N * nkb));
  uint8_t* sbb = xmalloc((size_t)(nnb * nkb));
  for (int64_t i = 0; i < M * nkb; ++i) sa[i] = (uint8_t)(120 + next32() % 15);
  for (int64_t i = 0; i < N * nkb; ++i) sbr[i] = (uint8_t)(120 + next32() % 15);
  for (int64_t i = 0; i < nnb * nkb; ++i) sbb[i] = (uint8_t)(120 + next32() % 15);
  double* y = xmalloc(sizeof(double) * (size_t)(M * N));
  double* t = xmalloc(sizeof(double) * (size_t)(M * N));
  orc_gemm(M, N, K, a, K, 0, sa, bnk, K, 1, 0, sbb, 0, 0, M, y, t, N);
  for (int64_t i = 0; i < M * N; ++i) CHECK(t[i] >= fabs(y[i]));
  uint8_t* sbbt = xmalloc((size_t)(nkb * nnb));
  for (int64_t kb = 0; kb < nkb; ++kb)
    for (int64_t nb = 0; nb < nnb; ++nb) sbbt[kb * nnb + nb] = sbb[nb * nkb + kb];
  double* y2 = xmalloc(sizeof(double) * (size_t)(M * N));
  orc_gemm(M, N, K, a, K, 0, sa, bkn, N, 1, 1, sbbt, 0, 0, M, y2, t, N);
  for (int64_t i = 0; i < M * N; ++i) CHECK(y2[i] == y[i]);
  orc_gemm(M, N, K, a, K, 0, sa, bnk, K, 1, 0, sbr, 1, 5, M - 3, y, t, N);
  int64_t ii[4] = {0, 5, 36, 17}, jj[4] = {0, 132, 1, 64};
  double ye[4], te[4];
  orc_gemm_elems(M, N, K, a, K, 0, sa, bnk, K, 1, 0, sbr, 1, ii, jj, 4, ye, te);
  float* fsa = xmalloc(sizeof(float) * (size_t)(M * nkb));
  float* fsb = xmalloc(sizeof(float) * (size_t)(N * nkb));
  for (int64_t i = 0; i < M * nkb; ++i) fsa[i] = (float)(0.5 + unif());
  for (int64_t i = 0; i < N * nkb; ++i) fsb[i] = (float)(0.5 + unif());
  orc_gemm_f32s(M, N, K, a, K, 0, fsa, bnk, K, 1, 0, fsb, 1, 0, M, y, t, N);
  orc_gemm_f32s_elems(M, N, K, a, K, 0, fsa, bkn, N, 1, 1, fsb, 0, ii, jj, 4, ye, te);
  uint8_t* msa = xmalloc((size_t)(M * (K / 32)));
  uint8_t* msb = xmalloc((size_t)(N * (K / 32)));
  for (int64_t i = 0; i < M * (K / 32); ++i) msa[i] = (uint8_t)(120 + next32() % 15);
  for (int64_t i = 0; i < N * (K / 32); ++i) msb[i] = (uint8_t)(120 + next32() % 15);
  orc_mx_gemm(M, N, K, a, K, 0, msa, bnk, K, 1, msb, 0, M, y, t, N);
  orc_mx_gemm_elems(M, N, K, a, K, 0, msa, bnk, K, 1, msb, ii, jj, 4, ye, te);
  free(a); free(bnk); free(bkn); free(sa); free(sbr); free(sbb); free(sbbt); free(y); free(y2); free(t);
  free(fsa); free(fsb); free(msa); free(msb);
}

static void gaussws(void) {
  const int64_t rows = 70, cols = 200, ld = 208;
  for (int dtype = 0; dtype < 2; ++dtype) {
    void* w = make_input(dtype, rows, cols, ld, -4);
    const int64_t nbr = (rows + 31) / 32, nbc = (cols + 31) / 32;
    int8_t* bt = xmalloc((size_t)(nbr * nbc));
    for (int64_t i = 0; i < nbr * nbc; ++i) bt[i] = (int8_t)((int)(next32() % 250) - 120);
    uint16_t* out = xmalloc(sizeof(uint16_t) * (size_t)(rows * cols));
    orc_gaussws(w, dtype, rows, cols, ld, bt, 1234, 5, out, cols, 0, nbr);
    int8_t* r = xmalloc((size_t)(rows * cols));
    orc_gaussws_noise(1234, 5, rows, cols, r);
    for (int64_t i = 0; i < rows * cols; ++i) CHECK(r[i] >= -2 && r[i] <= 2);
    free(w); free(bt); free(out); free(r);
  }
  uint64_t ctr[4] = {~0ull, ~0ull, 1, 2}, key[2] = {3, ~0ull}, o[4];
  orc_philox4x64(ctr, key, o);
  CHECK(orc_gaussws_r(0u) == 0 && orc_gaussws_r(0xFFFFFFFFu) == -2);
}

int main(void) {
  codec();
  quantizers();
  gemms();
  gaussws();
  if (fails) {
    fprintf(stderr, "%d oracle check(s) failed\n", fails);
    return 1;
  }
  printf("oracle driver: all checks passed\n");
  return 0;
}
