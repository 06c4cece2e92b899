// Shared device helpers for the gfx950 kernels of libmxq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"

namespace mxq {

// Size arithmetic of the host-side checks on caller-supplied (non-negative)
// sizes: the product or sum, or INT64_MAX when it does not fit, so that a
// limit check on the result rejects it instead of overflowing.
inline int64_t sat_mul(int64_t a, int64_t b) {
  int64_t r;
  return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}
inline int64_t sat_add(int64_t a, int64_t b) {
  int64_t r;
  return __builtin_add_overflow(a, b, &r) ? INT64_MAX : r;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// a and b rounded to BF16 (nearest even) by one packed conversion, a in the
// low half.  Converting each value on its own costs a conversion per value
// plus a shift and an OR per pair.
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

constexpr int kWave = 64;

// DPP quad permutations: exchange with lane^1 and lane^2 inside groups of 4.
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]

__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, int ctrl_xor1_or_2) {
  if (ctrl_xor1_or_2 == kQuadXor1)
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor1, 0xF, 0xF, false);
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor2, 0xF, 0xF, false);
}

// Packed max of the magnitudes of two BF16 values held in one dword.  The
// sign bits are cleared, so integer order equals magnitude order, and every
// NaN pattern (0x7F81..0x7FFF) compares above Inf (0x7F80) above all finite
// values: the maximum propagates NaN, then Inf.
__device__ __forceinline__ u16x2 absmax2(uint32_t a, uint32_t b) {
  u16x2 x = __builtin_bit_cast(u16x2, a & 0x7FFF7FFFu);
  u16x2 y = __builtin_bit_cast(u16x2, b & 0x7FFF7FFFu);
  return __builtin_elementwise_max(x, y);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// E8M0 scale code of an MX block from the largest BF16 magnitude pattern
// (sign cleared).  floor(log2(amax)) is the unbiased exponent field E - 127,
// so e = E - 127 - 8, clamped at -127: code = e + 127 = max(E - 8, 0).  BF16
// subnormals and zero (E == 0) give code 0; NaN/Inf give 0xFF.
__device__ __forceinline__ uint32_t mx_scale_code(uint32_t amax_bits) {
  uint32_t E = amax_bits >> 7;
  if (amax_bits >= 0x7F80u) return 0xFFu;
  return E > 8u ? E - 8u : 0u;
}

// 2^-e as FP32 for scale code c = e + 127 (c <= 253): exponent field 254 - c.
__device__ __forceinline__ float mx_inv_scale(uint32_t code) {
  return __builtin_bit_cast(float, (254u - code) << 23);
}

// Saturating round-to-nearest-even of two FP32 values to E4M3, packed into
// byte pair HI (false: bytes 0-1, true: bytes 2-3) of `old`.  The hardware
// conversion rounds to nearest even, including subnormals, but returns NaN
// instead of saturating at >= 464, so values are clamped to +-448 first.
template <bool HI>
__device__ __forceinline__ uint32_t cvt2_e4m3_sat(float a, float b, uint32_t old) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

}  // namespace mxq
