/*
 * oracle.h -- plain, slow CPU oracle for hybrid-granularity FP8 quantization
 * and the block-scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes,
 * links or calls this code; only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark do.  It shares no source with the HIP
 * path.
 *
 * Every value is computed in fp64 from the definitions on the pages; see the
 * comments in oracle.c for the passage each function follows.
 *
 * Integer conventions of this file (chosen here, independent of the library):
 *   fmt:    0 = E4M3, 1 = E5M2
 *   dtype:  0 = fp32, 1 = bf16 (raw 16-bit patterns)
 *   rule:   0 = round-up power-of-two scale, 1 = OCP floor(log2 amax) - emax
 *   b_layout: 0 = B stored [N][K] (K contiguous), 1 = B stored [K][N]
 *   b_scale:  0 = one scale per 128x128 tile of B's storage,
 *             1 = one scale per (column n, 128-wide K block)
 */
#ifndef MXFP8_ORACLE_H
#define MXFP8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

double orc_decode(int fmt, uint8_t code);
uint8_t orc_encode(int fmt, double x);
int orc_scale_exp_ceil(int fmt, double amax);
int orc_scale_exp_floor(int fmt, double amax);

void orc_quantize_rows(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                       int fmt, uint8_t* q, int64_t ldq, uint8_t* s);
void orc_quantize_cols_t(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                         int fmt, uint8_t* qt, int64_t ldq, uint8_t* st);
void orc_quantize_block(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw,
                        int fmt, uint8_t* q, int64_t ldq, uint8_t* s);
void orc_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                     int fmt, int rule, uint8_t* q, int64_t ldq, uint8_t* s, uint8_t* counts);

float orc_scale_f32(int fmt, float amax);
void orc_quantize_rows_f32s(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                            int fmt, uint8_t* q, int64_t ldq, float* s);
void orc_quantize_cols_t_f32s(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                              int fmt, uint8_t* qt, int64_t ldq, float* st);
void orc_quantize_block_f32s(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw,
                             int fmt, uint8_t* q, int64_t ldq, float* s);

void orc_gemm(int64_t M, int64_t N, int64_t K,
              const uint8_t* a, int64_t lda, int a_fmt, const uint8_t* sa,
              const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
              const uint8_t* sb, int b_scale,
              int64_t m0, int64_t m1, double* y, double* t, int64_t ldy);
void orc_gemm_elems(int64_t M, int64_t N, int64_t K,
                    const uint8_t* a, int64_t lda, int a_fmt, const uint8_t* sa,
                    const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
                    const uint8_t* sb, int b_scale,
                    const int64_t* ii, const int64_t* jj, int64_t n, double* y, double* t);

void orc_gemm_f32s(int64_t M, int64_t N, int64_t K,
                   const uint8_t* a, int64_t lda, int a_fmt, const float* sa,
                   const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
                   const float* sb, int b_scale,
                   int64_t m0, int64_t m1, double* y, double* t, int64_t ldy);
void orc_gemm_f32s_elems(int64_t M, int64_t N, int64_t K,
                         const uint8_t* a, int64_t lda, int a_fmt, const float* sa,
                         const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
                         const float* sb, int b_scale,
                         const int64_t* ii, const int64_t* jj, int64_t n, double* y, double* t);

void orc_mx_gemm(int64_t M, int64_t N, int64_t K,
                 const uint8_t* a, int64_t lda, int a_fmt, const uint8_t* sa,
                 const uint8_t* b, int64_t ldb, int b_fmt, const uint8_t* sb,
                 int64_t m0, int64_t m1, double* y, double* t, int64_t ldy);
void orc_mx_gemm_elems(int64_t M, int64_t N, int64_t K,
                       const uint8_t* a, int64_t lda, int a_fmt, const uint8_t* sa,
                       const uint8_t* b, int64_t ldb, int b_fmt, const uint8_t* sb,
                       const int64_t* ii, const int64_t* jj, int64_t n, double* y, double* t);

void orc_philox4x64(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);
int orc_gaussws_r(uint32_t u);
void orc_gaussws_noise(uint64_t seed, uint64_t stream, int64_t rows, int64_t cols, int8_t* r_out);
void orc_gaussws(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw, const int8_t* bt,
                 uint64_t seed, uint64_t stream, uint16_t* out, int64_t ldo, int64_t i0, int64_t i1);

void orc_decode_array(int fmt, const uint8_t* codes, int64_t n, double* out);
void orc_encode_array(int fmt, const double* x, int64_t n, uint8_t* out);
void orc_encode_f32_range(int fmt, uint32_t start, int64_t n, uint8_t* out);

#ifdef __cplusplus
}
#endif
#endif
