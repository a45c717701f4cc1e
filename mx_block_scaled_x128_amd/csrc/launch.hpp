// launch.hpp -- internal host launchers behind the C ABI (argument checking
// is done by the caller, api.cpp; these only size grids and launch).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace mxfp8 {

// Compute units of the current device (cached per device; concurrent first
// calls store the same value).
inline int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Whether a kernel streams its input with non-temporal loads: inputs of at
// least 64 MiB (a quarter of the 256 MB last-level cache), read once per call.
inline uint32_t stream_loads(int64_t rows, int64_t cols, int64_t elem_bytes) {
  return rows * cols * elem_bytes >= (int64_t(64) << 20) ? 1u : 0u;
}

// Token-wise 1x128 groups along rows.  cols % 16 == 0.
void launch_quant_row(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                      uint8_t* q, int64_t ldq, uint8_t* s, hipStream_t stream);
// 128-token groups down columns, transposed codes.  rows % 16 == 0, cols % 16 == 0.
void launch_quant_col_t(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                        uint8_t* qt, int64_t ldq, uint8_t* st, hipStream_t stream);
// 128x128 tiles.  cols % 16 == 0.
void launch_quant_block(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw, int fmt,
                        uint8_t* q, int64_t ldq, uint8_t* s, hipStream_t stream);
// fp32-scale variants of the three above (scales as floats, same layouts).
void launch_quant_row_f32s(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                           uint8_t* q, int64_t ldq, float* s, hipStream_t stream);
void launch_quant_col_t_f32s(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                             uint8_t* qt, int64_t ldq, float* st, hipStream_t stream);
void launch_quant_block_f32s(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw, int fmt,
                             uint8_t* q, int64_t ldq, float* s, hipStream_t stream);
// Both token orientations from one read: row groups (q, s) and transposed
// column groups (qt, st).  rows % 16 == 0, cols % 16 == 0.
void launch_quant_dual(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                       int64_t ldq, uint8_t* s, uint8_t* qt, int64_t ldqt, uint8_t* st, hipStream_t stream);
// 128x128 tiles, codes and transposed codes; s [rows/128][cols/128], st its transpose.
// rows % 16 == 0, cols % 16 == 0.
void launch_quant_block_dual(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw, int fmt,
                             uint8_t* q, int64_t ldq, uint8_t* s, uint8_t* qt, int64_t ldqt, uint8_t* st,
                             hipStream_t stream);
// 32-element MX blocks along rows.  cols % 32 == 0.
void launch_mx(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int fmt, int rule,
               uint8_t* q, int64_t ldq, uint8_t* s, uint8_t* counts, hipStream_t stream);
// Block-scaled GEMM.  K % 128 == 0, M, N >= 1.
void launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, int a_fmt,
                 const uint8_t* sa, const uint8_t* b, int64_t ldb, int b_fmt, int b_layout,
                 const uint8_t* sb, int b_scale_mode, void* c, int64_t ldc, int c_dtype,
                 hipStream_t stream);

// The block-scaled GEMM with fp32 scales (same layouts, floats).  K % 128 == 0,
// scale pointers 4-byte aligned.
void launch_gemm_f32s(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, int a_fmt,
                      const float* sa, const uint8_t* b, int64_t ldb, int b_fmt, int b_layout, const float* sb,
                      int b_scale_mode, void* c, int64_t ldc, int c_dtype, hipStream_t stream);

// MX GEMM: A [M][K] with scales [M][K/32], B [N][K] with scales [N][K/32].
// K % 128 == 0, M, N >= 1, scale pointers 4-byte aligned.
void launch_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, int a_fmt,
                    const uint8_t* sa, const uint8_t* b, int64_t ldb, int b_fmt, const uint8_t* sb, void* c,
                    int64_t ldc, int c_dtype, hipStream_t stream);

// GaussWS sampled weight (bf16 bits): 32x32 blocks, int8 bitwidth per block.
// cols % 8 == 0.
void launch_gaussws(const void* w, int dtype, int64_t rows, int64_t cols, int64_t ldw, const int8_t* bt,
                    uint64_t seed, uint64_t stream_id, uint16_t* out, int64_t ldo, hipStream_t stream);

}  // namespace mxfp8
