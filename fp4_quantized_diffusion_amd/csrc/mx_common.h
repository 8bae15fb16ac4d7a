// Device helpers shared by the MXFP4 quantizers and the GEMM epilogue that
// quantizes its own output: the GELU of the rollout's hidden activation
// (exact erf form, through erfc) and the MX block-scale / code rules.
// Both users must produce the same bits for the same input, so these are the
// only copies. Every function turns floating-point contraction off: each
// operation rounds on its own, whatever the including file's flags.
#pragma once
#include "common.h"

namespace fp4r {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// GELU(z) = z Phi(z), Phi the standard normal CDF, through the complementary
// error function: with Q = erfc(|z| / sqrt 2) / 2, Phi(z) = Q for z < 0 and
// 1 - Q otherwise, so the negative side never forms 1 + erf (which cancels
// to a few correct bits below z = -3). erfc uses the Chebyshev fit of Press
// et al., Numerical Recipes in C (2nd ed.), section 6.2 ("erfcc", fractional
// error below 1.2e-7 for x >= 0):
//     erfc(x) ~ t exp(-x^2 + P(t)),  t = 1 / (1 + x / 2),  P of degree 9.
// Here Q = t 2^(log2(e) P(t) - 1) 2^(-z^2 log2(e) / 2): the polynomial is
// evaluated with its coefficients scaled by log2(e) (and 1 taken off the
// constant term), and the large-argument factor takes the exact two-term
// split of z^2 and of log2(e) / 2 plus a first-order correction for the low
// parts, so it adds no rounding error of its own. v_rcp_f32 / v_exp_f32 are
// 1-ulp operations. Relative error of the result: about 5e-7 for |z| <= 12
// (fp32 emulation of this sequence against float64 erfc). |z| is clamped at
// 16, where Q is below fp32's range (Phi is then 0 or 1).
#define FP4R_L2E(c) ((float)((c) * 1.4426950408889634))
// Q(|z|) as above, for a = |z| >= 0.
__device__ __forceinline__ float phi_tail(float a_in) {
#pragma clang fp contract(off)
  constexpr float kHalfLog2eHi = -0.7213475f;     // -log2(e) / 2, high part
  constexpr float kHalfLog2eLo = -9.629815e-09f;  // and the rest
  constexpr float kLn2 = 0.693147180559945309f;
  const float a = __builtin_amdgcn_fmed3f(a_in, 0.0f, 16.0f);
  const float t = __builtin_amdgcn_rcpf(fmaf(a, 0.353553390593273762f, 1.0f));  // 1 / (1 + a / (2 sqrt 2))
  float p = FP4R_L2E(0.17087277);
  p = fmaf(p, t, FP4R_L2E(-0.82215223));
  p = fmaf(p, t, FP4R_L2E(1.48851587));
  p = fmaf(p, t, FP4R_L2E(-1.13520398));
  p = fmaf(p, t, FP4R_L2E(0.27886807));
  p = fmaf(p, t, FP4R_L2E(-0.18628806));
  p = fmaf(p, t, FP4R_L2E(0.09678418));
  p = fmaf(p, t, FP4R_L2E(0.37409196));
  p = fmaf(p, t, FP4R_L2E(1.00002368));
  p = fmaf(p, t, (float)(-1.26551223 * 1.4426950408889634 - 1.0));
  const float eph = __builtin_amdgcn_exp2f(p);    // exp(P(t)) / 2
  const float s = a * a, s_lo = fmaf(a, a, -s);  // a^2 = s + s_lo exactly
  const float y = s * kHalfLog2eHi;
  float e = fmaf(s, kHalfLog2eHi, -y);            // -a^2 log2(e) / 2 = y + e (to ~2^-48 relative)
  e = fmaf(s_lo, kHalfLog2eHi, e);
  e = fmaf(s, kHalfLog2eLo, e);
  float es = __builtin_amdgcn_exp2f(y);
  es = fmaf(es * e, kLn2, es);                     // exp2(y + e) ~ exp2(y) (1 + e ln 2)
  return t * (eph * es);
}
#undef FP4R_L2E

// z Phi(z) from q = Q(|z|): z q for z < 0 and z (1 - q) = z - |z| q for
// z >= 0, i.e. max(z, -0) - |z| q, formed by one fma (one rounding). The
// IEEE maximum (gfx950's v_maximum3_f32) orders -0 below +0, so the addend
// is -0 for every z <= -0 and the result keeps the sign of z, zeros and
// underflows included.
__device__ __forceinline__ float gelu_q(float z, float q) {
  return fmaf(-fabsf(z), q, __builtin_elementwise_maximum(z, -0.0f));
}

__device__ __forceinline__ float gelu_erfc(float z) {
  return gelu_q(z, phi_tail(fabsf(z)));
}

// The standard normal density phi(a) = exp(-a^2 / 2) / sqrt(2 pi), with the
// exponent split exactly as in phi_tail (relative error a few fp32 ulps).
__device__ __forceinline__ float gauss_pdf(float a) {
#pragma clang fp contract(off)
  constexpr float kHalfLog2eHi = -0.7213475f;
  constexpr float kHalfLog2eLo = -9.629815e-09f;
  constexpr float kLn2 = 0.693147180559945309f;
  constexpr float kInvSqrt2Pi = 0.398942280401432678f;
  const float s = a * a, s_lo = fmaf(a, a, -s);
  const float y = s * kHalfLog2eHi;
  float e = fmaf(s, kHalfLog2eHi, -y);
  e = fmaf(s_lo, kHalfLog2eHi, e);
  e = fmaf(s, kHalfLog2eLo, e);
  float es = __builtin_amdgcn_exp2f(y);
  es = fmaf(es * e, kLn2, es);
  return es * kInvSqrt2Pi;
}

// GELU of a bf16 input through a table of Q(|z|). A bf16 value has 8
// significant bits, so the magnitudes 2^-22 .. 16 are 26 binades of 128
// values plus 16 itself: 3329 entries (13 KiB in LDS), holding phi_tail of
// exactly those values, so gelu_q(z, table entry) is bit-identical to
// gelu_erfc(z) for 2^-22 <= |z| <= 16, and beyond 16 too, because phi_tail
// clamps |z| at 16. Below 2^-22 the index clamps to the 2^-22 entry: Phi
// there differs from Phi(z) by less than 0.4 * 2^-22 (2e-7 relative).
constexpr uint32_t kGeluLo = (127u - 22u) << 7;  // bf16 magnitude bits of 2^-22
constexpr uint32_t kGeluHi = (127u + 4u) << 7;   // and of 16
constexpr int kGeluTab = (int)(kGeluHi - kGeluLo + 1);

// Fill the table (every thread of the workgroup takes a share; the caller
// synchronizes before any other wave reads it).
__device__ __forceinline__ void gelu_table_fill(float* tab) {
  for (int e = threadIdx.x; e < kGeluTab; e += blockDim.x)
    tab[e] = phi_tail(__uint_as_float((kGeluLo + (uint32_t)e) << 16));
}

__device__ __forceinline__ float gelu_bf16(float z, const float* tab) {
  const uint32_t m = min(max((__float_as_uint(z) >> 16) & 0x7FFFu, kGeluLo), kGeluHi);  // z is a bf16 value
  return gelu_q(z, tab[m - kGeluLo]);
}

// GELU of an fp32 input through a table of (Q(a), phi(a)) at the bf16
// magnitudes a from 2^-10 to 16: 14 binades of 128 values plus 16 itself,
// 1793 entries (14 KiB in LDS), Q = phi_tail(a). With a_c the bf16 rounding
// of |z| clamped to [2^-10, 16] and d = |z| - a_c (half a bf16 ulp above
// 2^-10, |d| <= 2^-8 a_c; |d| <= 2^-10 below; exact by Sterbenz where
// |z| >= a_c / 2), the fourth-order Taylor expansion
//     Q(a_c + d) = Q - phi d [1 - a_c d / 2 + (a_c^2 - 1) d^2 / 6
//                             + a_c (3 - a_c^2) d^3 / 24]
// follows from Q^(1) = -phi, Q^(2) = a phi, Q^(3) = (1 - a^2) phi,
// Q^(4) = (a^3 - 3 a) phi. What it leaves out, about
// phi (a^4 - 6 a^2 + 3) d^5 / 120, is below 6e-8 of Q for |z| <= 6 (largest
// just below 6; below 2e-10 for |z| <= 4; a float64 evaluation of the
// expansion at 4 million points against erfc gives 5.5e-8); the rounding of
// the expansion adds a few fp32 ulps of phi d, so the result carries
// phi_tail's error (about 5e-7 relative). At the table's points (d = 0) the
// result is phi_tail's, bit for bit. Beyond |z| = kGeluTaylorMax the callers
// take gelu_erfc instead, element by element, so the value depends on z
// alone.
constexpr uint32_t kGeluTLo = (127u - 10u) << 7;  // bf16 magnitude bits of 2^-10
constexpr int kGeluTTab = (int)(kGeluHi - kGeluTLo + 1);
constexpr float kGeluTaylorMax = 6.0f;

// Entries above kGeluTaylorMax are (0, 0): the exact treatment never reads
// them (it evaluates erfc there), and with them the expansion gives exactly
// z for z > 6 and -0 for z < -6 (see gelu_f32_expand).
__device__ __forceinline__ void gelu_table_fill(float2* tab) {
  for (int e = threadIdx.x; e < kGeluTTab; e += blockDim.x) {
    const float a = __uint_as_float((kGeluTLo + (uint32_t)e) << 16);
    tab[e] = a <= kGeluTaylorMax ? make_float2(phi_tail(a), gauss_pdf(a)) : make_float2(0.0f, 0.0f);
  }
}

// pat: the bit pattern of the bf16 rounding (nearest even) of |z| in the
// upper half of the word, the lower half zero, so that it reads as that
// value in fp32; clamped, it is a_c itself and, shifted, the table index.
// The bracket of the expansion above is evaluated in x = a_c d,
//     1 - x/2 + x^2/6 - x^3/24 + d^2 (x/8 - 1/6),
// the same polynomial term by term (a_c d^2 = x d, a_c^2 d^2 = x^2,
// a_c^3 d^3 = x^3). gelu_f32_from is valid for |z| <= kGeluTaylorMax.
__device__ __forceinline__ uint32_t gelu_tab_clamp(uint32_t pat) {
  return min(max(pat, kGeluTLo << 16), kGeluHi << 16);  // any pattern, NaN included, stays in the table
}
__device__ __forceinline__ float2 gelu_tab_entry(uint32_t pat, const float2* tab) {
  return tab[(gelu_tab_clamp(pat) >> 16) - kGeluTLo];
}
__device__ __forceinline__ float gelu_f32_from(float z, uint32_t pat, float2 t) {
#pragma clang fp contract(off)
  const float ac = __uint_as_float(gelu_tab_clamp(pat));
  const float d = fabsf(z) - ac;
  const float x = ac * d;
  float b = fmaf(fmaf(fmaf(x, -1.0f / 24.0f, 1.0f / 6.0f), x, -0.5f), x, 1.0f);
  b = fmaf(d * d, fmaf(x, 0.125f, -1.0f / 6.0f), b);
  return gelu_q(z, fmaf(-t.y, b * d, t.x));
}

// GELU of N (even) fp32 values through the table, in parts so that a
// caller can issue the table reads of one batch before it evaluates the
// previous one: gelu_f32_fetch forms the indices and issues the reads;
// gelu_f32_finish evaluates the expansion where |z| <= kGeluTaylorMax and
// the evaluated erfc elsewhere (a branch that lanes skip unless one of their
// N values is that large or NaN: the IEEE maximum propagates NaN). A caller
// that keeps that branch out of its main sequence takes gelu_f32_expand
// instead and redoes with gelu_f32_finish wherever the difference can show
// (see gelu_f32_expand). The bf16 roundings come from the hardware's
// nearest-even pair conversion.
template <int N>
struct GeluBatch {
  float z[N];
  uint32_t p[N];
  float2 t[N];
  float m;
};

// MAX: also form b.m, the batch's largest |z| (NaN if any z is), which
// gelu_f32_tail and gelu_f32_finish read.
template <int N, bool MAX = true>
__device__ __forceinline__ void gelu_f32_fetch(GeluBatch<N>& b, const float2* tab) {
  b.m = 0.0f;
#pragma unroll
  for (int e = 0; e < N; e += 2) {
    uint32_t u = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)b.z[e], (__bf16)b.z[e + 1]});
    asm("" : "+v"(u));  // one pair conversion
    u &= 0x7FFF7FFFu;   // the magnitudes (nearest-even rounding is symmetric)
    b.p[e] = u << 16;
    b.p[e + 1] = u & 0xFFFF0000u;
    if (MAX) b.m = __builtin_elementwise_maximum(b.m, __builtin_elementwise_maximum(fabsf(b.z[e]), fabsf(b.z[e + 1])));
  }
#pragma unroll
  for (int e = 0; e < N; ++e) b.t[e] = gelu_tab_entry(b.p[e], tab);
}

// The expansion for every value, whatever its size: the exact treatment
// where gelu_f32_tail(b) is false. Beyond |z| = kGeluTaylorMax it gives, in
// fp32: z itself for z > 6, as the evaluated erfc does (z Q(z) is below
// half an ulp of z); for z < -6 a negative value of magnitude below 6e-9
// (|z| < 6.016, which takes the entry of 6) or -0 (the entries above 6 are
// zero), where the evaluated erfc gives a negative value below 6e-9 or -0;
// and NaN for NaN or infinite z and once the expansion overflows (|z|
// beyond about 1e9).
template <int N>
__device__ __forceinline__ void gelu_f32_expand(float* g, const GeluBatch<N>& b) {
#pragma unroll
  for (int e = 0; e < N; ++e) g[e] = gelu_f32_from(b.z[e], b.p[e], b.t[e]);
}

template <int N>
__device__ __forceinline__ bool gelu_f32_tail(const GeluBatch<N>& b) {
  return !(b.m <= kGeluTaylorMax);  // NaN too
}

template <int N>
__device__ __forceinline__ void gelu_f32_finish(float* g, const GeluBatch<N>& b) {
  gelu_f32_expand(g, b);
  if (gelu_f32_tail(b)) {
    // One evaluation per trip of a loop that stays rolled, so the code stays
    // small wherever this is inlined; the value is picked out and put back
    // by selects on compile-time positions (no register array is indexed
    // by a run-time value, which would move it to scratch memory).
#pragma unroll 1
    for (int e = 0; e < N; ++e) {
      float ze = b.z[0];
#pragma unroll
      for (int k = 1; k < N; ++k) ze = k == e ? b.z[k] : ze;
      const float r = gelu_erfc(ze);
      const bool tail = !(fabsf(ze) <= kGeluTaylorMax);
#pragma unroll
      for (int k = 0; k < N; ++k) g[k] = (k == e && tail) ? r : g[k];
    }
  }
}

template <int N>
__device__ __forceinline__ void gelu_f32_tab_n(float* g, const float* z, const float2* tab) {
  GeluBatch<N> b;
#pragma unroll
  for (int e = 0; e < N; ++e) b.z[e] = z[e];
  gelu_f32_fetch(b, tab);
  gelu_f32_finish(g, b);
}

// Bits of max |v_j| by the IEEE maximum (v_maximum3_f32, absolute values as
// source modifiers): for non-NaN inputs the bits of the largest magnitude,
// and a NaN input gives a NaN, whose exponent field, like that of every
// larger-than-finite value, is all ones. mx_scale reads only the exponent
// field, so it sees what the maximum of the bit patterns (sign cleared)
// would give.
template <int N>
__device__ __forceinline__ uint32_t amax_bits(const float* v) {
  float m = fabsf(v[0]);
#pragma unroll
  for (int j = 1; j < N; ++j) m = __builtin_elementwise_maximum(m, fabsf(v[j]));
  return __float_as_uint(m);
}

__device__ __forceinline__ uint32_t amax_bits8(const float v[8]) { return amax_bits<8>(v); }

// MX: E8M0 scale byte and the packed codes of one octet, given the block amax bits.
// S = max(biased_exponent(amax) - 2, 0) is floor(log2 amax) - 2 + 127 clamped at
// E = -127 (zero and subnormal amax land on the clamp). The codes encode
// x * 2^(127 - S); on the ALU path the multiplier is a normal power of two and
// the product is exact wherever it can reach a non-zero code.
__device__ __forceinline__ uint32_t mx_scale(uint32_t amax_bits) {
  int s = (int)(amax_bits >> 23) - 2;
  return (uint32_t)(s < 0 ? 0 : s);
}

__device__ __forceinline__ uint32_t mx_pack8_alu(const float v[8], uint32_t S) {
#pragma clang fp contract(off)
  const float mul = __uint_as_float((254u - S) << 23);
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) w |= e2m1_nibble(v[j] * mul) << (4 * j);
  return w;
}

// Same codes through gfx950's V_CVT_SCALEF32_PK_FP4_F32, which converts
// x / scale to E2M1 with round-to-nearest-even, saturation at 6 and the sign
// kept -- checked against the oracle over millions of fp32 inputs and four
// power-of-two scales, and by the exhaustive element-rounding sweep test.
// Byte j of the result takes elements 2j (low nibble) and 2j + 1. Blocks with
// S <= 2 take the ALU path: S = 0 would need a subnormal scale, and for
// S = 1, 2 the block can hold fp32 subnormals that must round to non-zero
// codes (|x| in (2^(S - 129), 2^-126)), which the ALU path's exact
// power-of-two product handles by construction. Such blocks (amax below
// 2^-122) do not occur in practice, so the branch costs one compare.
// mx_pack8_hw is the converter alone, for callers that have set such blocks
// aside (S > 2).
__device__ __forceinline__ uint32_t mx_pack8_hw(const float v[8], uint32_t S) {
  const float sc = __uint_as_float(S << 23);  // 2^(S - 127)
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], sc, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], sc, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], sc, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], sc, 3);
  return w;
}

__device__ __forceinline__ uint32_t mx_pack8(const float v[8], uint32_t S) {
  return S <= 2 ? mx_pack8_alu(v, S) : mx_pack8_hw(v, S);
}

}  // namespace fp4r
