// Device helpers shared by the VC-Attention HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vc.h"

namespace vc {

constexpr int kD = 128;      // head dim (the only one built)
constexpr int kBlock = 128;  // hardware block of V-Smooth: 128 tokens

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// float32 -> OCP E4M3 byte, round to nearest even, saturating at +-448.  The
// hardware conversion rounds to nearest even but turns |x| >= 464 into NaN, so
// the input is clamped to the largest finite E4M3 value first (fmaxf/fminf keep
// the sign of -0).
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float x) {
  float c = fminf(fmaxf(x, -448.0f), 448.0f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0u, false) & 0xFFu;
}

// Two floats -> two E4M3 bytes in the low (kHi=false) or high 16 bits of `old`.
template <bool kHi>
__device__ __forceinline__ uint32_t pack2_e4m3_sat(float a, float b, uint32_t old) {
  float ca = fminf(fmaxf(a, -448.0f), 448.0f);
  float cb = fminf(fmaxf(b, -448.0f), 448.0f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, old, kHi);
}

// E4M3 byte -> float (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

// 32-bit float atomic max for non-negative values (bit patterns order like ints).
__device__ __forceinline__ void atomic_max_nonneg(float* addr, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

}  // namespace vc

// Host-side status helpers (defined in api.cpp).
int vc_set_hip_error(int hip_error);
