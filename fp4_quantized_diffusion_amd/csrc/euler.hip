// Explicit Euler update of the sampler's ODE, x_out = x + dt * v, for gfx950.
// The rollout takes 6 steps from t = 1 to t = 0 (aitrends summary of Sol-RL,
// Stage-1 paragraph). Pure HBM stream: 12 bytes per element with fp32 v
// (10 with bf16 v); 16-byte vector loads/stores, grid-stride.
#include "common.h"

namespace fp4r {
namespace {

constexpr int kThreads = 256;

// Each thread issues the loads of kUnroll grid-stride iterations before it
// uses the first, so that every wave keeps 2 x kUnroll 16-byte loads in
// flight; x_out is written once and not read back by this kernel
// (non-temporal stores).
constexpr int kUnroll = 4;

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int BF16>
__device__ __forceinline__ float4 load_v4(const void* v, int64_t i) {
  if (BF16) {
    const uint2 q = reinterpret_cast<const uint2*>(v)[i];
    return make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xFFFF0000u), __uint_as_float(q.y << 16),
                       __uint_as_float(q.y & 0xFFFF0000u));
  }
  return reinterpret_cast<const float4*>(v)[i];
}

// x_out may be x (in place): each element is read, then written, by one
// thread, so x carries no __restrict__.
template <int BF16>
__global__ __launch_bounds__(kThreads) void euler_kernel(float* x_out, const float* x, const void* __restrict__ v,
                                                         int64_t numel, float dt) {
  const int64_t n4 = numel >> 2;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; i0 < n4; i0 += kUnroll * stride) {
    float4 a[kUnroll], b[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n4) {
        a[u] = reinterpret_cast<const float4*>(x)[i];
        b[u] = load_v4<BF16>(v, i);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n4) {
        const f32x4 o = {fmaf(dt, b[u].x, a[u].x), fmaf(dt, b[u].y, a[u].y), fmaf(dt, b[u].z, a[u].z),
                         fmaf(dt, b[u].w, a[u].w)};
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(x_out) + i);
      }
    }
  }
  // ragged tail (numel % 4 elements), handled by the first threads of block 0
  if (blockIdx.x == 0 && threadIdx.x < (numel & 3)) {
    const int64_t j = (n4 << 2) + threadIdx.x;
    const float vb = BF16 ? __uint_as_float(((uint32_t)reinterpret_cast<const uint16_t*>(v)[j]) << 16)
                          : reinterpret_cast<const float*>(v)[j];
    x_out[j] = fmaf(dt, vb, x[j]);
  }
}

}  // namespace

hipError_t launch_euler(float* x_out, const float* x, const void* v, int v_bf16, int64_t numel,
                        float t_cur, float t_next, hipStream_t st) {
  const float dt = t_next - t_cur;  // fp32 subtraction on the host (IEEE single)
  int64_t g = ((numel >> 2) + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  if (g > 8192) g = 8192;
  if (v_bf16)
    euler_kernel<1><<<(unsigned)g, kThreads, 0, st>>>(x_out, x, v, numel, dt);
  else
    euler_kernel<0><<<(unsigned)g, kThreads, 0, st>>>(x_out, x, v, numel, dt);
  return hipGetLastError();
}

}  // namespace fp4r
