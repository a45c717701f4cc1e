// Host-only driver for the C ABI's argument validation (api.cpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer.  The HIP launchers and
// hipGetLastError are replaced by stubs that record their calls, so every
// entry point runs its checks and, for valid arguments, reaches its launcher
// without a GPU.  Fake pointers are never dereferenced by the validation.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "mxfp8.h"

namespace {
int g_calls = 0;
int64_t g_last[4] = {0, 0, 0, 0};
int g_fail = 0;
void rec(int64_t a, int64_t b, int64_t c, int64_t d) {
  ++g_calls;
  g_last[0] = a;
  g_last[1] = b;
  g_last[2] = c;
  g_last[3] = d;
}
}  // namespace

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

namespace mxfp8 {
void launch_quant_row(const void*, int, int64_t r, int64_t c, int64_t ld, int, uint8_t*, int64_t lq, uint8_t*, hipStream_t) { rec(r, c, ld, lq); }
void launch_quant_col_t(const void*, int, int64_t r, int64_t c, int64_t ld, int, uint8_t*, int64_t lq, uint8_t*, hipStream_t) { rec(r, c, ld, lq); }
void launch_quant_block(const void*, int, int64_t r, int64_t c, int64_t ld, int, uint8_t*, int64_t lq, uint8_t*, hipStream_t) { rec(r, c, ld, lq); }
void launch_quant_row_f32s(const void*, int, int64_t r, int64_t c, int64_t ld, int, uint8_t*, int64_t lq, float*, hipStream_t) { rec(r, c, ld, lq); }
void launch_quant_col_t_f32s(const void*, int, int64_t r, int64_t c, int64_t ld, int, uint8_t*, int64_t lq, float*, hipStream_t) { rec(r, c, ld, lq); }
void launch_quant_block_f32s(const void*, int, int64_t r, int64_t c, int64_t ld, int, uint8_t*, int64_t lq, float*, hipStream_t) { rec(r, c, ld, lq); }
void launch_quant_dual(const void*, int, int64_t r, int64_t c, int64_t ld, int, uint8_t*, int64_t lq, uint8_t*, uint8_t*, int64_t, uint8_t*, hipStream_t) { rec(r, c, ld, lq); }
void launch_quant_block_dual(const void*, int, int64_t r, int64_t c, int64_t ld, int, uint8_t*, int64_t lq, uint8_t*, uint8_t*, int64_t, uint8_t*, hipStream_t) { rec(r, c, ld, lq); }
void launch_mx(const void*, int, int64_t r, int64_t c, int64_t ld, int, int, uint8_t*, int64_t lq, uint8_t*, uint8_t*, hipStream_t) { rec(r, c, ld, lq); }
void launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t*, int64_t, int, const uint8_t*, const uint8_t*, int64_t, int, int, const uint8_t*, int, void*, int64_t ldc, int, hipStream_t) { rec(M, N, K, ldc); }
void launch_gemm_f32s(int64_t M, int64_t N, int64_t K, const uint8_t*, int64_t, int, const float*, const uint8_t*, int64_t, int, int, const float*, int, void*, int64_t ldc, int, hipStream_t) { rec(M, N, K, ldc); }
void launch_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t*, int64_t, int, const uint8_t*, const uint8_t*, int64_t, int, const uint8_t*, void*, int64_t ldc, int, hipStream_t) { rec(M, N, K, ldc); }
void launch_gaussws(const void*, int, int64_t r, int64_t c, int64_t ld, const int8_t*, uint64_t, uint64_t, uint16_t*, int64_t lo, hipStream_t) { rec(r, c, ld, lo); }
}  // namespace mxfp8

#define EXPECT(expr, want)                                                                  \
  do {                                                                                      \
    const int got_ = (expr);                                                                \
    if (got_ != (want)) {                                                                   \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #expr, got_, \
                   (int)(want));                                                            \
      ++g_fail;                                                                             \
    }                                                                                       \
  } while (0)

// Valid call: status OK and exactly one launcher call with these leading arguments.
#define LAUNCHES(expr, a, b, c, d)                                                              \
  do {                                                                                          \
    const int before_ = g_calls;                                                                \
    EXPECT(expr, MXFP8_OK);                                                                     \
    if (g_calls != before_ + 1 || g_last[0] != (a) || g_last[1] != (b) || g_last[2] != (c) ||  \
        g_last[3] != (d)) {                                                                     \
      std::fprintf(stderr, "line %d: %s did not reach its launcher as expected\n", __LINE__, #expr); \
      ++g_fail;                                                                                 \
    }                                                                                           \
  } while (0)

#define P(v) reinterpret_cast<uint8_t*>(static_cast<uintptr_t>(v))
#define F(v) reinterpret_cast<float*>(static_cast<uintptr_t>(v))

int main() {
  const uintptr_t X = 0x100000, Q = 0x200000, S = 0x300000, C = 0x400000, T = 0x500000, U = 0x600000;
  const uintptr_t MIS = 0x200008;
  void* st = nullptr;
  // token quantizer
  LAUNCHES(fp8_quantize_token(P(X), 1, 256, 512, 512, 0, 0, P(Q), 512, P(S), st), 256, 512, 512, 512);
  LAUNCHES(fp8_quantize_token(P(X), 0, 256, 512, 512, 1, 1, P(Q), 256, P(S), st), 256, 512, 512, 256);
  EXPECT(fp8_quantize_token(P(X), 2, 256, 512, 512, 0, 0, P(Q), 512, P(S), st), MXFP8_ERR_ENUM);
  EXPECT(fp8_quantize_token(P(X), 1, -1, 512, 512, 0, 0, P(Q), 512, P(S), st), MXFP8_ERR_SHAPE);
  EXPECT(fp8_quantize_token(P(X), 1, INT64_MAX, 512, 512, 0, 0, P(Q), 512, P(S), st), MXFP8_ERR_SHAPE);
  EXPECT(fp8_quantize_token(nullptr, 1, 0, 512, 512, 0, 0, nullptr, 512, nullptr, st), MXFP8_OK);
  EXPECT(fp8_quantize_token(nullptr, 1, 256, 512, 512, 0, 0, P(Q), 512, P(S), st), MXFP8_ERR_NULL);
  EXPECT(fp8_quantize_token(P(X), 1, 256, 512, 500, 0, 0, P(Q), 512, P(S), st), MXFP8_ERR_LD);
  EXPECT(fp8_quantize_token(P(X), 1, 256, 512, INT64_MAX, 0, 0, P(Q), 512, P(S), st), MXFP8_ERR_LD);
  EXPECT(fp8_quantize_token(P(MIS), 1, 256, 512, 512, 0, 0, P(Q), 512, P(S), st), MXFP8_ERR_ALIGN);
  EXPECT(fp8_quantize_token(P(X), 1, 256, 512, 512, 0, 0, P(X), 512, P(S), st), MXFP8_ERR_ALIAS);
  EXPECT(fp8_quantize_token(P(X), 1, 136, 512, 512, 1, 0, P(Q), 144, P(S), st), MXFP8_ERR_SHAPE);
  // block quantizer and the fp32-scale variants
  LAUNCHES(fp8_quantize_block(P(X), 0, 300, 512, 512, 1, P(Q), 512, P(S), st), 300, 512, 512, 512);
  EXPECT(fp8_quantize_block(P(X), 0, 300, 24, 32, 1, P(Q), 32, P(S), st), MXFP8_ERR_SHAPE);
  EXPECT(fp8_quantize_block(P(X), 0, 300, 512, 512, 1, P(X), 512, P(S), st), MXFP8_ERR_ALIAS);
  LAUNCHES(fp8_quantize_token_f32s(P(X), 1, 64, 256, 256, 0, 0, P(Q), 256, F(S), st), 64, 256, 256, 256);
  EXPECT(fp8_quantize_token_f32s(P(X), 1, 64, 256, 256, 0, 0, P(Q), 256, F(S + 2), st), MXFP8_ERR_ALIGN);
  LAUNCHES(fp8_quantize_block_f32s(P(X), 1, 64, 256, 256, 0, P(Q), 256, F(S), st), 64, 256, 256, 256);
  // two-orientation quantizers
  LAUNCHES(fp8_quantize_token_dual(P(X), 1, 256, 128, 128, 0, P(Q), 128, P(S), P(T), 256, P(U), st), 256, 128, 128, 128);
  EXPECT(fp8_quantize_token_dual(P(X), 1, 256, 128, 128, 0, P(Q), 128, P(S), P(Q), 256, P(U), st), MXFP8_ERR_ALIAS);
  EXPECT(fp8_quantize_token_dual(P(X), 1, 250, 128, 128, 0, P(Q), 128, P(S), P(T), 256, P(U), st), MXFP8_ERR_SHAPE);
  LAUNCHES(fp8_quantize_block_dual(P(X), 1, 256, 128, 128, 0, P(Q), 128, P(S), P(T), 256, P(U), st), 256, 128, 128, 128);
  // MX quantizer
  LAUNCHES(mx_quantize(P(X), 0, 64, 96, 96, 0, 1, P(Q), 96, P(S), P(C), st), 64, 96, 96, 96);
  EXPECT(mx_quantize(P(X), 0, 64, 80, 80, 0, 1, P(Q), 80, P(S), P(C), st), MXFP8_ERR_SHAPE);
  EXPECT(mx_quantize(P(X), 0, 64, 96, 96, 0, 2, P(Q), 96, P(S), P(C), st), MXFP8_ERR_ENUM);
  EXPECT(mx_quantize(P(X), 0, 64, 96, 96, 0, 1, P(Q), 96, P(S), P(Q), st), MXFP8_ERR_ALIAS);
  // block-scaled GEMM
  LAUNCHES(fp8_block_scaled_gemm(200, 300, 512, P(X), 512, 0, P(S), P(Q), 512, 1, 0, P(T), 0, P(C), 304, 1, st), 200, 300, 512, 304);
  LAUNCHES(fp8_block_scaled_gemm(200, 300, 512, P(X), 512, 0, P(S), P(Q), 304, 1, 1, P(T), 0, P(C), 304, 0, st), 200, 300, 512, 304);
  LAUNCHES(fp8_block_scaled_gemm(64, 48, 0, nullptr, 0, 0, nullptr, nullptr, 0, 0, 0, nullptr, 0, P(C), 48, 0, st), 64, 48, 0, 48);
  EXPECT(fp8_block_scaled_gemm(200, 300, 500, P(X), 512, 0, P(S), P(Q), 512, 1, 0, P(T), 0, P(C), 304, 1, st), MXFP8_ERR_SHAPE);
  EXPECT(fp8_block_scaled_gemm(200, 300, 512, P(X), 512, 0, P(S), P(Q), 512, 1, 1, P(T), 1, P(C), 304, 1, st), MXFP8_ERR_ENUM);
  EXPECT(fp8_block_scaled_gemm(200, 300, 512, P(X), 512, 0, P(S), P(Q), int64_t(1) << 25, 1, 0, P(T), 0, P(C), 304, 1, st), MXFP8_ERR_LD);
  EXPECT(fp8_block_scaled_gemm(INT64_MAX, 300, 512, P(X), 512, 0, P(S), P(Q), 512, 1, 0, P(T), 0, P(C), 304, 1, st), MXFP8_ERR_SHAPE);
  EXPECT(fp8_block_scaled_gemm(200, 300, 512, P(X), 512, 0, P(S), P(Q), 512, 1, 0, P(T), 0, P(X), 304, 1, st), MXFP8_ERR_ALIAS);
  LAUNCHES(fp8_gemm_f32s(128, 128, 256, P(X), 256, 0, F(S), P(Q), 256, 0, 0, F(T), 1, P(C), 128, 0, st), 128, 128, 256, 128);
  EXPECT(fp8_gemm_f32s(128, 128, 256, P(X), 256, 0, F(S + 1), P(Q), 256, 0, 0, F(T), 1, P(C), 128, 0, st), MXFP8_ERR_ALIGN);
  LAUNCHES(mx_gemm(128, 96, 256, P(X), 256, 1, P(S), P(Q), 256, 0, P(T), P(C), 96, 1, st), 128, 96, 256, 96);
  EXPECT(mx_gemm(128, 96, 256, P(X), 256, 1, P(S + 2), P(Q), 256, 0, P(T), P(C), 96, 1, st), MXFP8_ERR_ALIGN);
  // GaussWS
  LAUNCHES(gaussws_sample(P(X), 0, 40, 64, 64, reinterpret_cast<int8_t*>(S), 1, 2, reinterpret_cast<uint16_t*>(C), 64, st), 40, 64, 64, 64);
  EXPECT(gaussws_sample(P(X), 0, 40, 60, 64, reinterpret_cast<int8_t*>(S), 1, 2, reinterpret_cast<uint16_t*>(C), 64, st), MXFP8_ERR_SHAPE);
  // status strings
  for (int s = -3; s < 12; ++s)
    if (!mxfp8_status_string(s)) ++g_fail;
  EXPECT(mxfp8_version(), MXFP8_VERSION);
  if (g_fail) {
    std::fprintf(stderr, "%d ABI check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("abi driver: all checks passed (%d launcher calls)\n", g_calls);
  return 0;
}
