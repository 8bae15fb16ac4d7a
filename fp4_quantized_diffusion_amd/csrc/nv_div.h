// The correctly rounded quotient fl(x / d) of the NVFP4-style quantizers,
// without a division per element: with y = fl(1 / d) computed once per block
// (a correctly rounded division), q = fl(x y) and then twice
// q <- fl(q + fl(x - d q) y) with fmas. The first correction leaves q within
// one ulp of x / d (faithful); with y correctly rounded and q faithful, the
// remainder x - d q is exact and the second correction gives the correctly
// rounded quotient (Markstein, IBM J. Res. Dev. 34(1), 1990; Muller et al.,
// Handbook of Floating-Point Arithmetic, "Newton-Raphson based division with
// an FMA"). It holds while the intermediates stay normal and finite, which
// nv_div_applies secures (d in [2^-100, 2^100], |x| / d <= 2^64) wherever the
// quotient reaches 2^-3, the smallest magnitude that can round to a non-zero
// E2M1 code. Below that a subnormal x can make the remainder underflow and
// the last bits differ from IEEE division; such quotients encode to a signed
// zero either way. The quotient takes the sign of x explicitly: for x = -0
// the corrections would add +0 to -0 and give +0.
//
// Plain C++ apart from the HIP function qualifiers, so that a host build of
// this very sequence can be checked against IEEE division on the CPU.
#pragma once

namespace fp4r {

__host__ __device__ inline bool nv_div_applies(float d, float amax, float y) {
  return d >= 0x1p-100f && d <= 0x1p100f && amax * y <= 0x1p64f;
}

__host__ __device__ inline float nv_div(float x, float d, float y) {
#pragma clang fp contract(off)
  float q = x * y;
  q = fmaf(fmaf(-d, q, x), y, q);
  return __builtin_copysignf(fmaf(fmaf(-d, q, x), y, q), x);
}

}  // namespace fp4r
