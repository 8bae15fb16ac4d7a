// Device helpers shared by the elementwise quantizers (quant.hip) and the
// LoRA-merge quantizer (lora.hip): the octet load and the 4-lane MX block.
#pragma once
#include "mx_common.h"

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

}  // namespace fp4r
