// Device helpers shared by the elementwise quantizers (quant.hip) and the
// LoRA-merge quantizer (lora.hip): the octet load, the 4-lane MX block and
// the 2-lane NVFP4-style block. Both users must produce the same bits for
// the same input, so these are the only copies.
#pragma once
#include "mx_common.h"
#include "nv_div.h"

namespace fp4r {

// Eight consecutive elements of a row (an "octet") as fp32: one 16-byte
// load; bf16 widens exactly.
template <int BF16>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float v[8]) {
  if (BF16) {
    uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Block scale of a 32-block held as 4 octets in lanes 4q..4q+3, and the
// octet's code word.
__device__ __forceinline__ uint32_t mx_block(const float v[8], uint32_t& S) {
  uint32_t am = amax_bits8(v);
  am = max(am, (uint32_t)__shfl_xor((int)am, 1));
  am = max(am, (uint32_t)__shfl_xor((int)am, 2));
  S = mx_scale(am);
  return mx_pack8(v, S);
}


// E4M3 (bias 7, max 448) code of a non-negative finite fp32 value, round to
// nearest even, saturating at 448 (code 0x7E).
__device__ __forceinline__ uint32_t e4m3_rne(float s) {
#pragma clang fp contract(off)
  const uint32_t b = __float_as_uint(s);
  const int e = (int)(b >> 23) - 127;
  if (e < -6) {
    // below the smallest normal 2^-6: steps of 2^-9; s * 512 is exact
    return (uint32_t)rintf(s * 512.0f);  // 0..8 (8 is the smallest normal, code 0x08)
  }
  // round the 23-bit mantissa to 3 bits (nearest even), carry into the exponent
  const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;
  const uint32_t code = r - (120u << 3);  // exponent bias 127 -> 7
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_value(uint32_t S) {
#pragma clang fp contract(off)
  const uint32_t e = S >> 3, m = S & 7u;
  return e == 0 ? (float)m * 0x1p-9f : ldexpf((float)(8u + m), (int)e - 10);
}

// Raise an NVFP4-style amax word (the float bits of a non-negative value,
// ordered like integers) to at least t with an integer atomicMax. Most
// workgroups finish below the running maximum, so the word is read first and
// the atomic skipped then; the word only grows, so a stale read can only
// cost an atomic that was not needed. Without the check the same-address
// atomics of a few thousand workgroups serialize (2048 workgroups over a
// 36864 x 3072 bf16 activation: 129 -> 123 us for the whole quantization).
__device__ __forceinline__ void amax_raise(float* word, uint32_t t) {
  unsigned int* w = reinterpret_cast<unsigned int*>(word);
  if (t > __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(w, t);
}

// NVFP4-style block rule for one octet of a 16-block (the block's other
// octet in the adjacent lane, lane ^ 1; both lanes must call this together):
// block amax, s_f = fl(amax / tau) with tau = fl(6 sg), S = E4M3 code of s_f
// (nearest even, saturating at 448), d = fl(dec(S) sg), and the packed E2M1
// codes of fl(x / d) -- signed zeros for a block whose d is 0. sg is the
// tensor scale (positive).
//
// fl(x / d) is correctly rounded: nv_div (reciprocal once per block, two fma
// corrections) wherever nv_div_applies -- every block whose tensor scale
// comes from the data, where amax / d is at most about 6.4 -- and a plain
// division for other blocks (a caller-supplied tensor scale far from the
// data, NaN or infinite input). The codes come from the same scaled convert
// as the MX path, with scale 1.
__device__ __forceinline__ uint32_t nv_block(const float v[8], float sg, float tau, uint32_t& S) {
#pragma clang fp contract(off)
  uint32_t am = amax_bits8(v);
  am = max(am, (uint32_t)__shfl_xor((int)am, 1));  // the 2 octets of a 16-block
  const float sf = __uint_as_float(am) / tau;
  S = e4m3_rne(sf);
  const float d = e4m3_value(S) * sg;
  uint32_t w = 0;
  if (d == 0.0f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= ((__float_as_uint(v[j]) >> 28) & 8u) << (4 * j);
    return w;
  }
  float q[8];
  const float y = 1.0f / d;
  if (nv_div_applies(d, __uint_as_float(am), y)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = nv_div(v[j], d, y);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = v[j] / d;
  }
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[0], q[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
  return w;
}

}  // namespace fp4r
