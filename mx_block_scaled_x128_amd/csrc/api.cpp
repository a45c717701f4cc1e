// api.cpp -- the C ABI of libmxfp8 (declared in include/mxfp8.h): host-side
// argument validation, then dispatch to the HIP launchers.  Validation runs
// before any HIP call, so every error path can be exercised without a GPU.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/mxfp8.h"
#include "launch.hpp"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The GEMM kernels address an operand tile as a base plus 32-bit per-lane
// offsets of up to 255 rows times the leading dimension.
constexpr int64_t kMaxGemmLd = int64_t(1) << 24;

// Shared checks for the quantizers' input / code tensors.
int check_tensor_pair(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, const uint8_t* q,
                      int64_t ldq, int64_t q_row_len, const void* scales) {
  if (dtype != MXFP8_F32 && dtype != MXFP8_BF16) return MXFP8_ERR_ENUM;
  if (rows < 0 || cols < 0) return MXFP8_ERR_SHAPE;
  if (rows > INT32_MAX || cols > INT32_MAX) return MXFP8_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MXFP8_OK;
  if (!x || !q || !scales) return MXFP8_ERR_NULL;
  if (ldx < cols || ldx % 16 != 0) return MXFP8_ERR_LD;
  if (ldq < q_row_len || ldq % 16 != 0) return MXFP8_ERR_LD;
  if (!aligned16(x) || !aligned16(q)) return MXFP8_ERR_ALIGN;
  if ((const void*)q == x || scales == x || (const void*)q == scales) return MXFP8_ERR_ALIAS;
  return MXFP8_OK;
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MXFP8_OK : MXFP8_ERR_DEVICE;
}

}  // namespace

extern "C" {

int fp8_quantize_token(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int axis,
                       int fmt, uint8_t* q, int64_t ldq, uint8_t* scales, void* stream) {
  if (axis != MXFP8_GROUP_ROW && axis != MXFP8_GROUP_COL_T) return MXFP8_ERR_ENUM;
  if (fmt != MXFP8_E4M3 && fmt != MXFP8_E5M2) return MXFP8_ERR_ENUM;
  const int64_t q_row_len = axis == MXFP8_GROUP_ROW ? cols : rows;
  int st = check_tensor_pair(x, x_dtype, rows, cols, ldx, q, ldq, q_row_len, scales);
  if (st != MXFP8_OK || rows == 0 || cols == 0) return st;
  if (cols % 16 != 0) return MXFP8_ERR_SHAPE;
  if (axis == MXFP8_GROUP_COL_T && rows % 16 != 0) return MXFP8_ERR_SHAPE;
  (void)hipGetLastError();  // clear any stale error so the launch status is ours
  if (axis == MXFP8_GROUP_ROW)
    mxfp8::launch_quant_row(x, x_dtype, rows, cols, ldx, fmt, q, ldq, scales, (hipStream_t)stream);
  else
    mxfp8::launch_quant_col_t(x, x_dtype, rows, cols, ldx, fmt, q, ldq, scales, (hipStream_t)stream);
  return launch_status();
}

int fp8_quantize_block(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ldw, int fmt,
                       uint8_t* q, int64_t ldq, uint8_t* scales, void* stream) {
  if (fmt != MXFP8_E4M3 && fmt != MXFP8_E5M2) return MXFP8_ERR_ENUM;
  int st = check_tensor_pair(w, w_dtype, rows, cols, ldw, q, ldq, cols, scales);
  if (st != MXFP8_OK || rows == 0 || cols == 0) return st;
  if (cols % 16 != 0) return MXFP8_ERR_SHAPE;
  (void)hipGetLastError();
  mxfp8::launch_quant_block(w, w_dtype, rows, cols, ldw, fmt, q, ldq, scales, (hipStream_t)stream);
  return launch_status();
}

int fp8_quantize_token_f32s(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int axis,
                            int fmt, uint8_t* q, int64_t ldq, float* scales, void* stream) {
  if (axis != MXFP8_GROUP_ROW && axis != MXFP8_GROUP_COL_T) return MXFP8_ERR_ENUM;
  if (fmt != MXFP8_E4M3 && fmt != MXFP8_E5M2) return MXFP8_ERR_ENUM;
  const int64_t q_row_len = axis == MXFP8_GROUP_ROW ? cols : rows;
  int st = check_tensor_pair(x, x_dtype, rows, cols, ldx, q, ldq, q_row_len, scales);
  if (st != MXFP8_OK || rows == 0 || cols == 0) return st;
  if (cols % 16 != 0) return MXFP8_ERR_SHAPE;
  if (axis == MXFP8_GROUP_COL_T && rows % 16 != 0) return MXFP8_ERR_SHAPE;
  if ((uintptr_t)scales & 3) return MXFP8_ERR_ALIGN;
  (void)hipGetLastError();
  if (axis == MXFP8_GROUP_ROW)
    mxfp8::launch_quant_row_f32s(x, x_dtype, rows, cols, ldx, fmt, q, ldq, scales, (hipStream_t)stream);
  else
    mxfp8::launch_quant_col_t_f32s(x, x_dtype, rows, cols, ldx, fmt, q, ldq, scales, (hipStream_t)stream);
  return launch_status();
}

int fp8_quantize_block_f32s(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ldw, int fmt,
                            uint8_t* q, int64_t ldq, float* scales, void* stream) {
  if (fmt != MXFP8_E4M3 && fmt != MXFP8_E5M2) return MXFP8_ERR_ENUM;
  int st = check_tensor_pair(w, w_dtype, rows, cols, ldw, q, ldq, cols, scales);
  if (st != MXFP8_OK || rows == 0 || cols == 0) return st;
  if (cols % 16 != 0) return MXFP8_ERR_SHAPE;
  if ((uintptr_t)scales & 3) return MXFP8_ERR_ALIGN;
  (void)hipGetLastError();
  mxfp8::launch_quant_block_f32s(w, w_dtype, rows, cols, ldw, fmt, q, ldq, scales, (hipStream_t)stream);
  return launch_status();
}

namespace {
// Checks shared by the two-orientation quantizers: both output pairs as for
// the one-orientation calls, both extents multiples of 16, four distinct outputs.
static int check_dual(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt, const uint8_t* q,
               int64_t ldq, const uint8_t* s, const uint8_t* qt, int64_t ldqt, const uint8_t* st) {
  if (fmt != MXFP8_E4M3 && fmt != MXFP8_E5M2) return MXFP8_ERR_ENUM;
  int r = check_tensor_pair(x, dtype, rows, cols, ldx, q, ldq, cols, s);
  if (r != MXFP8_OK || rows == 0 || cols == 0) return r;
  r = check_tensor_pair(x, dtype, rows, cols, ldx, qt, ldqt, rows, st);
  if (r != MXFP8_OK) return r;
  if (cols % 16 != 0 || rows % 16 != 0) return MXFP8_ERR_SHAPE;
  if (q == qt || q == st || s == qt || s == st) return MXFP8_ERR_ALIAS;
  return MXFP8_OK;
}
}  // namespace

int fp8_quantize_token_dual(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                            uint8_t* q, int64_t ldq, uint8_t* scales, uint8_t* qt, int64_t ldqt,
                            uint8_t* scales_t, void* stream) {
  const int st = check_dual(x, x_dtype, rows, cols, ldx, fmt, q, ldq, scales, qt, ldqt, scales_t);
  if (st != MXFP8_OK || rows == 0 || cols == 0) return st;
  (void)hipGetLastError();
  mxfp8::launch_quant_dual(x, x_dtype, rows, cols, ldx, fmt, q, ldq, scales, qt, ldqt, scales_t,
                           (hipStream_t)stream);
  return launch_status();
}

int fp8_quantize_block_dual(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ldw, int fmt,
                            uint8_t* q, int64_t ldq, uint8_t* scales, uint8_t* qt, int64_t ldqt,
                            uint8_t* scales_t, void* stream) {
  const int st = check_dual(w, w_dtype, rows, cols, ldw, fmt, q, ldq, scales, qt, ldqt, scales_t);
  if (st != MXFP8_OK || rows == 0 || cols == 0) return st;
  (void)hipGetLastError();
  mxfp8::launch_quant_block_dual(w, w_dtype, rows, cols, ldw, fmt, q, ldq, scales, qt, ldqt, scales_t,
                                 (hipStream_t)stream);
  return launch_status();
}

int mx_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt, int rule,
                uint8_t* q, int64_t ldq, uint8_t* scales, uint8_t* clamp_counts, void* stream) {
  if (fmt != MXFP8_E4M3 && fmt != MXFP8_E5M2) return MXFP8_ERR_ENUM;
  if (rule != MXFP8_RULE_CEIL && rule != MXFP8_RULE_FLOOR) return MXFP8_ERR_ENUM;
  int st = check_tensor_pair(x, x_dtype, rows, cols, ldx, q, ldq, cols, scales);
  if (st != MXFP8_OK || rows == 0 || cols == 0) return st;
  if (cols % 32 != 0) return MXFP8_ERR_SHAPE;
  if (clamp_counts && ((const void*)clamp_counts == x || clamp_counts == q || clamp_counts == scales))
    return MXFP8_ERR_ALIAS;
  (void)hipGetLastError();
  mxfp8::launch_mx(x, x_dtype, rows, cols, ldx, fmt, rule, q, ldq, scales, clamp_counts, (hipStream_t)stream);
  return launch_status();
}

int fp8_block_scaled_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, int a_fmt,
                          const uint8_t* a_scales, const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
                          const uint8_t* b_scales, int b_scale_mode, void* c, int64_t ldc, int c_dtype,
                          void* stream) {
  if (a_fmt != MXFP8_E4M3 && a_fmt != MXFP8_E5M2) return MXFP8_ERR_ENUM;
  if (b_fmt != MXFP8_E4M3 && b_fmt != MXFP8_E5M2) return MXFP8_ERR_ENUM;
  if (b_layout != MXFP8_B_NK && b_layout != MXFP8_B_KN) return MXFP8_ERR_ENUM;
  if (b_scale_mode != MXFP8_SCALE_BLOCK128 && b_scale_mode != MXFP8_SCALE_ROW128) return MXFP8_ERR_ENUM;
  if (b_layout == MXFP8_B_KN && b_scale_mode == MXFP8_SCALE_ROW128) return MXFP8_ERR_ENUM;
  if (c_dtype != MXFP8_F32 && c_dtype != MXFP8_BF16) return MXFP8_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0) return MXFP8_ERR_SHAPE;
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return MXFP8_ERR_SHAPE;
  if (K % 128 != 0) return MXFP8_ERR_SHAPE;
  if (M == 0 || N == 0) return MXFP8_OK;
  if (!c) return MXFP8_ERR_NULL;
  if (K > 0 && (!a || !a_scales || !b || !b_scales)) return MXFP8_ERR_NULL;
  if (ldc < N || ldc % 16 != 0) return MXFP8_ERR_LD;
  if (K > 0) {
    if (lda < K || lda % 16 != 0) return MXFP8_ERR_LD;
    const int64_t b_row = b_layout == MXFP8_B_NK ? K : N;
    if (ldb < b_row || ldb % 16 != 0) return MXFP8_ERR_LD;
    if (lda > kMaxGemmLd || ldb > kMaxGemmLd) return MXFP8_ERR_LD;
    if (!aligned16(a) || !aligned16(b)) return MXFP8_ERR_ALIGN;
  }
  if (!aligned16(c)) return MXFP8_ERR_ALIGN;
  if (c == (const void*)a || c == (const void*)b || c == (const void*)a_scales || c == (const void*)b_scales)
    return MXFP8_ERR_ALIAS;
  (void)hipGetLastError();
  mxfp8::launch_gemm(M, N, K, a, lda, a_fmt, a_scales, b, ldb, b_fmt, b_layout, b_scales, b_scale_mode, c, ldc,
                     c_dtype, (hipStream_t)stream);
  return launch_status();
}

int fp8_gemm_f32s(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, int a_fmt, const float* a_scales,
                  const uint8_t* b, int64_t ldb, int b_fmt, int b_layout, const float* b_scales, int b_scale_mode,
                  void* c, int64_t ldc, int c_dtype, void* stream) {
  if (a_fmt != MXFP8_E4M3 && a_fmt != MXFP8_E5M2) return MXFP8_ERR_ENUM;
  if (b_fmt != MXFP8_E4M3 && b_fmt != MXFP8_E5M2) return MXFP8_ERR_ENUM;
  if (b_layout != MXFP8_B_NK && b_layout != MXFP8_B_KN) return MXFP8_ERR_ENUM;
  if (b_scale_mode != MXFP8_SCALE_BLOCK128 && b_scale_mode != MXFP8_SCALE_ROW128) return MXFP8_ERR_ENUM;
  if (b_scale_mode == MXFP8_SCALE_ROW128 && b_layout != MXFP8_B_NK) return MXFP8_ERR_ENUM;
  if (c_dtype != MXFP8_F32 && c_dtype != MXFP8_BF16) return MXFP8_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0) return MXFP8_ERR_SHAPE;
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return MXFP8_ERR_SHAPE;
  if (K % 128 != 0) return MXFP8_ERR_SHAPE;
  if (M == 0 || N == 0) return MXFP8_OK;
  if (!c) return MXFP8_ERR_NULL;
  if (K > 0 && (!a || !a_scales || !b || !b_scales)) return MXFP8_ERR_NULL;
  if (ldc < N || ldc % 16 != 0) return MXFP8_ERR_LD;
  if (K > 0) {
    if (lda < K || lda % 16 != 0) return MXFP8_ERR_LD;
    const int64_t b_row = b_layout == MXFP8_B_NK ? K : N;
    if (ldb < b_row || ldb % 16 != 0) return MXFP8_ERR_LD;
    if (lda > kMaxGemmLd || ldb > kMaxGemmLd) return MXFP8_ERR_LD;
    if (!aligned16(a) || !aligned16(b)) return MXFP8_ERR_ALIGN;
    if (((uintptr_t)a_scales & 3) || ((uintptr_t)b_scales & 3)) return MXFP8_ERR_ALIGN;
  }
  if (!aligned16(c)) return MXFP8_ERR_ALIGN;
  if (c == (const void*)a || c == (const void*)b || c == (const void*)a_scales || c == (const void*)b_scales)
    return MXFP8_ERR_ALIAS;
  (void)hipGetLastError();
  mxfp8::launch_gemm_f32s(M, N, K, a, lda, a_fmt, a_scales, b, ldb, b_fmt, b_layout, b_scales, b_scale_mode, c,
                          ldc, c_dtype, (hipStream_t)stream);
  return launch_status();
}

int mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, int a_fmt, const uint8_t* a_scales,
            const uint8_t* b, int64_t ldb, int b_fmt, const uint8_t* b_scales, void* c, int64_t ldc, int c_dtype,
            void* stream) {
  if (a_fmt != MXFP8_E4M3 && a_fmt != MXFP8_E5M2) return MXFP8_ERR_ENUM;
  if (b_fmt != MXFP8_E4M3 && b_fmt != MXFP8_E5M2) return MXFP8_ERR_ENUM;
  if (c_dtype != MXFP8_F32 && c_dtype != MXFP8_BF16) return MXFP8_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0) return MXFP8_ERR_SHAPE;
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return MXFP8_ERR_SHAPE;
  if (K % 128 != 0) return MXFP8_ERR_SHAPE;
  if (M == 0 || N == 0) return MXFP8_OK;
  if (!c) return MXFP8_ERR_NULL;
  if (K > 0 && (!a || !a_scales || !b || !b_scales)) return MXFP8_ERR_NULL;
  if (ldc < N || ldc % 16 != 0) return MXFP8_ERR_LD;
  if (K > 0) {
    if (lda < K || lda % 16 != 0) return MXFP8_ERR_LD;
    if (ldb < K || ldb % 16 != 0) return MXFP8_ERR_LD;
    if (lda > kMaxGemmLd || ldb > kMaxGemmLd) return MXFP8_ERR_LD;
    if (!aligned16(a) || !aligned16(b)) return MXFP8_ERR_ALIGN;
    if (((uintptr_t)a_scales & 3) || ((uintptr_t)b_scales & 3)) return MXFP8_ERR_ALIGN;
  }
  if (!aligned16(c)) return MXFP8_ERR_ALIGN;
  if (c == (const void*)a || c == (const void*)b || c == (const void*)a_scales || c == (const void*)b_scales)
    return MXFP8_ERR_ALIAS;
  (void)hipGetLastError();
  mxfp8::launch_mx_gemm(M, N, K, a, lda, a_fmt, a_scales, b, ldb, b_fmt, b_scales, c, ldc, c_dtype,
                        (hipStream_t)stream);
  return launch_status();
}

int gaussws_sample(const void* w, int w_dtype, int64_t rows, int64_t cols, int64_t ldw, const int8_t* bitwidths,
                   uint64_t seed, uint64_t stream_id, uint16_t* w_hat, int64_t ldo, void* stream) {
  if (w_dtype != MXFP8_F32 && w_dtype != MXFP8_BF16) return MXFP8_ERR_ENUM;
  if (rows < 0 || cols < 0) return MXFP8_ERR_SHAPE;
  if (rows > INT32_MAX / 2 || cols > INT32_MAX / 2) return MXFP8_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MXFP8_OK;
  if (!w || !bitwidths || !w_hat) return MXFP8_ERR_NULL;
  if (ldw < cols || ldw % 16 != 0) return MXFP8_ERR_LD;
  if (ldo < cols || ldo % 16 != 0) return MXFP8_ERR_LD;
  if (cols % 8 != 0) return MXFP8_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(w_hat)) return MXFP8_ERR_ALIGN;
  if ((const void*)w_hat == w || (const void*)w_hat == (const void*)bitwidths) return MXFP8_ERR_ALIAS;
  (void)hipGetLastError();
  mxfp8::launch_gaussws(w, w_dtype, rows, cols, ldw, bitwidths, seed, stream_id, w_hat, ldo, (hipStream_t)stream);
  return launch_status();
}

const char* mxfp8_status_string(int status) {
  switch (status) {
    case MXFP8_OK: return "ok";
    case MXFP8_ERR_NULL: return "a required pointer is NULL";
    case MXFP8_ERR_SHAPE: return "extent negative, too large, or not a multiple the entry point requires";
    case MXFP8_ERR_LD: return "leading dimension smaller than the row or not a multiple of 16 elements";
    case MXFP8_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case MXFP8_ERR_ENUM: return "enum argument out of range or unsupported combination";
    case MXFP8_ERR_ALIAS: return "an output pointer equals an input pointer";
    case MXFP8_ERR_DEVICE: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int mxfp8_version(void) { return MXFP8_VERSION; }

}  // extern "C"
