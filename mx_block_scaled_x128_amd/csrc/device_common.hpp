// device_common.hpp -- gfx950 device helpers shared by the quantizer and GEMM
// kernels: the FP8 cast, power-of-two scale exponents from fp32 bit fields,
// and wavefront reductions.
//
// Formats [FP8 Formats for Deep Learning, "Core claim"]: E4M3 (bias 7, no
// infinities, largest finite 448 = 1.75 * 2^8) and E5M2 (bias 15, IEEE
// specials, largest finite 57344 = 1.75 * 2^15), OCP encodings.  The
// hardware cast v_cvt_pk_{fp8,bf8}_f32 rounds to nearest even, keeps the sign
// of zero and handles subnormal results; it does NOT saturate (finite
// overflow becomes NaN / inf), so callers clamp wherever a scaled value can
// exceed the largest finite value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp8 {

// Largest finite value and its binade exponent q (fmax = 1.75 * 2^q).
template <int FMT> struct FmtInfo;
template <> struct FmtInfo<0> { static constexpr int q = 8;  static constexpr float fmax = 448.0f; };
template <> struct FmtInfo<1> { static constexpr int q = 15; static constexpr float fmax = 57344.0f; };

// Round-up power-of-two scale exponent ["A Comprehensive FP8 Training Recipe
// ...", "What carries the argument": the UE8M0 scale is rounded up so the
// scaled group never leaves the FP8 range]: the smallest integer e with
// amax <= fmax * 2^e, clamped to [-127, 127], amax == 0 -> -127.
// With amax = (1 + M/2^23) * 2^p (normal, biased exponent E >= 1) and
// fmax = 1.75 * 2^q: amax <= 1.75 * 2^p exactly when M <= 0.75 * 2^23, so
// e = p - q when M <= 0x600000 and p - q + 1 otherwise.  A subnormal amax
// (E == 0) is below fmax * 2^-127 for both formats, so e = -127.
template <int FMT>
__device__ __forceinline__ int scale_exp_ceil(uint32_t amax_bits) {
  const int E = (int)(amax_bits >> 23);
  const uint32_t M = amax_bits & 0x7FFFFFu;
  int e = E - 127 - FmtInfo<FMT>::q + (M > 0x600000u ? 1 : 0);
  e = (E == 0) ? -127 : e;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// OCP MX shared exponent ["Characterization and Mitigation of Training
// Instabilities in Microscaling Formats", "What carries the argument"]:
// X = floor(log2 amax) - q, clamped to [-127, 127]; amax == 0 (and any
// subnormal amax, whose floor(log2) is below -126) -> -127.
template <int FMT>
__device__ __forceinline__ int scale_exp_floor(uint32_t amax_bits) {
  const int E = (int)(amax_bits >> 23);
  int e = E - 127 - FmtInfo<FMT>::q;
  e = (E == 0) ? -127 : e;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^-e as an fp32 for e in [-127, 126] (always a normal number).  The
// exponents above never exceed 120 for finite fp32 inputs.
__device__ __forceinline__ float pow2_neg(int e) {
  return __uint_as_float((uint32_t)(127 - e) << 23);
}

// fp32 group scale of the "FP8 with an FP32 scale" variant (named as a
// Table 4 variant on the review page of "A Comprehensive FP8 Training Recipe
// for Reasoning-Enhanced Language Models", not defined there; read as):
// amax / fmax in IEEE single precision (HIP's default division is the
// correctly rounded one), 1 where that quotient rounds to zero.
template <int FMT>
__device__ __forceinline__ float scale_f32(uint32_t amax_bits) {
  const float s = __uint_as_float(amax_bits) / FmtInfo<FMT>::fmax;
  return s == 0.0f ? 1.0f : s;
}

// Four values -> four codes packed little-endian (a in the lowest byte).
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int w;
  if constexpr (FMT == 0) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

// bf16 pair (one dword) -> two fp32 values, exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// DPP controls (gfx9): quad permutations, rotations within a 16-lane row,
// mirror within each half row of 8 lanes.
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_ROR4 = 0x124;   // row_ror:4
constexpr int DPP_ROW_ROR8 = 0x128;   // row_ror:8
constexpr int DPP_HALF_MIRROR = 0x141;  // row_half_mirror

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
  return v > o ? v : o;
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_add(uint32_t v) {
  return v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Max of non-negative fp32 bit patterns (their integer order equals their
// value order) over aligned groups of 4, 8 or 16 lanes; every lane of the
// group receives the result.  All 64 lanes must be active.
__device__ __forceinline__ uint32_t max_quad(uint32_t v) {
  v = dpp_max<DPP_QUAD_XOR1>(v);
  return dpp_max<DPP_QUAD_XOR2>(v);
}
__device__ __forceinline__ uint32_t max_oct(uint32_t v) {
  return dpp_max<DPP_HALF_MIRROR>(max_quad(v));
}
__device__ __forceinline__ uint32_t max_row16(uint32_t v) {
  v = max_quad(v);
  v = dpp_max<DPP_ROW_ROR4>(v);
  return dpp_max<DPP_ROW_ROR8>(v);
}
__device__ __forceinline__ uint32_t max_wave(uint32_t v) {
  v = max_row16(v);
  uint32_t o = (uint32_t)__shfl_xor((int)v, 16);
  v = v > o ? v : o;
  o = (uint32_t)__shfl_xor((int)v, 32);
  return v > o ? v : o;
}
__device__ __forceinline__ uint32_t sum_quad(uint32_t v) {
  v = dpp_add<DPP_QUAD_XOR1>(v);
  return dpp_add<DPP_QUAD_XOR2>(v);
}

__device__ __forceinline__ uint32_t abs_bits(float f) { return __float_as_uint(f) & 0x7FFFFFFFu; }

// Loads of 8 consecutive input elements as fp32 (16 B for bf16, 32 B for fp32).
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));

// Code stores.  Ordinary (cache-allocating) stores, not non-temporal ones:
// the GEMM that follows a quantizer then reads its operands from the
// last-level cache.  Measured per step (quantizers + GEMM): dgrad 3 %, wgrad
// 5 % faster, although non-temporal stores make the tile quantizers alone
// 10-25 % faster.
__device__ __forceinline__ void store_codes(uint8_t* p, uint2 v) {
  *reinterpret_cast<nt_u32x2*>(p) = nt_u32x2{v.x, v.y};
}
__device__ __forceinline__ void store_codes(uint8_t* p, uint4 v) {
  *reinterpret_cast<nt_u32x4*>(p) = nt_u32x4{v.x, v.y, v.z, v.w};
}

// Eight input elements as fp32.  NT: a non-temporal load, which passes the
// caches without displacing their lines.  The 1x128 and 128x128 quantizers
// and the sampler read inputs of 64 MiB or more that way (a template choice
// per launch): an input read once then leaves the last-level cache to the
// codes just written, which the GEMM reads next (measured in the step: dgrad
// 2 %, the two-orientation quantizers 6 %, the sampler 3 % faster); smaller
// inputs, which stay cached from one step to the next, keep ordinary loads
// (the row quantizer of the fprop-sized workload is 6 % faster with them).
template <bool NT>
__device__ __forceinline__ void load8(const uint16_t* p, float (&f)[8]) {
  const nt_u32x4 v = NT ? __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p))
                        : *reinterpret_cast<const nt_u32x4*>(p);
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
template <bool NT>
__device__ __forceinline__ void load8(const float* p, float (&f)[8]) {
  const nt_f32x4 a = NT ? __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p))
                        : *reinterpret_cast<const nt_f32x4*>(p);
  const nt_f32x4 b = NT ? __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p + 4))
                        : *reinterpret_cast<const nt_f32x4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

}  // namespace mxfp8
