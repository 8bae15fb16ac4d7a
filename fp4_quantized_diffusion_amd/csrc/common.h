// Shared device helpers and host launch declarations of the fp4rollout library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common_host.h"

namespace fp4r {

// ---- device helpers ----
// f(std::integral_constant<int, I>) for I = B .. E-1, expanded at compile time
// (the index is a constant in every copy, whatever the body holds).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// Magnitude index of the nearest-even E2M1 value to a (a >= 0, finite or +inf).
// Decision points between neighbours, each tie going to the even index.
__device__ __forceinline__ uint32_t e2m1_index(float a) {
  uint32_t m = 0;
  m += (a > 0.25f);
  m += (a >= 0.75f);
  m += (a > 1.25f);
  m += (a >= 1.75f);
  m += (a > 2.5f);
  m += (a >= 3.5f);
  m += (a > 5.0f);
  return m;
}

// Signed E2M1 nibble of y (sign bit always kept, also for -0 and underflow).
__device__ __forceinline__ uint32_t e2m1_nibble(float y) {
  uint32_t s = (__float_as_uint(y) >> 28) & 8u;
  return s | e2m1_index(fabsf(y));
}

}  // namespace fp4r
