// DiffusionNFT pieces of the policy update on the regenerated samples, for
// gfx950: forward noising of the clean latents and the implicit
// positive/negative branch loss (VeRL-Omni DiffusionNFT docs, "Algorithm";
// the seeds the FP4 rollout selects are regenerated in BF16 and trained on
// with DiffusionNFT -- aitrends summary, Stage-2 paragraph).
//
//   x_t = (1 - t) x0 + t eps,        v = eps - x0 (the path's velocity),
//   v+ = (1 - beta) v_old + beta v_theta,  v- = (1 + beta) v_old - beta v_theta,
//   term_i = r_i ||v+ - v||^2 + (1 - r_i) ||v- - v||^2,   loss = mean_i term_i.
//
// Both are HBM streams (float4 per lane). The loss splits each sample over
// kSlices workgroups, each writing the two sums (||v+ - v||^2 and
// ||v- - v||^2) of its slice to a caller workspace; one workgroup then adds a
// sample's slices in a fixed order, forms term_i and, in the last step, the
// mean -- no atomics, so repeated calls give the same bits. Compiled with
// -ffp-contract=off: every rounding is the written one.
#include "common.h"

namespace fp4r {
namespace {

constexpr int kThreads = 256;
constexpr int kSlices = 64;  // workgroups per sample

// x_t = fma(t, eps, (1 - t) x0), one float4 per lane per step; workgroup
// (slice s, sample i) as in the loss, so t_i is one scalar load.
__global__ __launch_bounds__(kThreads) void nft_noise_kernel(const float4* __restrict__ x0,
                                                             const float4* __restrict__ eps,
                                                             const float* __restrict__ t, int64_t d4,
                                                             float4* __restrict__ xt) {
  const int64_t base = (int64_t)blockIdx.y * d4;
  const float ti = t[blockIdx.y], si = 1.0f - ti;
  for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < d4; j += (int64_t)kSlices * kThreads) {
    const float4 a = x0[base + j], e = eps[base + j];
    xt[base + j] = make_float4(fmaf(ti, e.x, si * a.x), fmaf(ti, e.y, si * a.y), fmaf(ti, e.z, si * a.z),
                               fmaf(ti, e.w, si * a.w));
  }
}

// Block-wide sum of two values in a fixed order (shuffle tree, then waves in order).
__device__ __forceinline__ void block_sum2(float& a, float& b, float* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh[2 * w] = a;
    sh[2 * w + 1] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a = b = 0.0f;
    for (int i = 0; i < kThreads / 64; ++i) {
      a += sh[2 * i];
      b += sh[2 * i + 1];
    }
  }
}

// Workgroup (slice s, sample i): sums over float4 groups s*kThreads + tid,
// stepping by kSlices*kThreads, of the sample's d4 groups.
__global__ __launch_bounds__(kThreads) void nft_loss_partial_kernel(
    const float4* __restrict__ vo, const float4* __restrict__ vt, const float4* __restrict__ x0,
    const float4* __restrict__ eps, float beta, int64_t d4, float* __restrict__ partials) {
  __shared__ float sh[2 * (kThreads / 64)];
  const int64_t i = blockIdx.y;
  const int64_t base = i * d4;
  const float bp = 1.0f - beta, bn = 1.0f + beta;
  float sp = 0.0f, sn = 0.0f;
  for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < d4; j += (int64_t)kSlices * kThreads) {
    const float4 o = vo[base + j], th = vt[base + j], a = x0[base + j], e = eps[base + j];
    const float ov[4] = {o.x, o.y, o.z, o.w}, tv[4] = {th.x, th.y, th.z, th.w};
    const float av[4] = {a.x, a.y, a.z, a.w}, ev[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float v = ev[c] - av[c];
      const float dp = (bp * ov[c] + beta * tv[c]) - v;
      const float dn = (bn * ov[c] - beta * tv[c]) - v;
      sp = fmaf(dp, dp, sp);
      sn = fmaf(dn, dn, sn);
    }
  }
  block_sum2(sp, sn, sh);
  if (threadIdx.x == 0) {
    partials[(i * kSlices + blockIdx.x) * 2] = sp;
    partials[(i * kSlices + blockIdx.x) * 2 + 1] = sn;
  }
}

// One workgroup: term_i = r_i P_i + (1 - r_i) N_i from the slices in order,
// then loss = (sum of terms in order) / n.
__global__ __launch_bounds__(kThreads) void nft_loss_final_kernel(const float* __restrict__ partials,
                                                                  const float* __restrict__ r, int64_t n,
                                                                  float* __restrict__ terms, float* __restrict__ loss) {
  __shared__ float sh[2 * (kThreads / 64)];
  for (int64_t i = 0; i < n; ++i) {
    float p = 0.0f, q = 0.0f;
    if (threadIdx.x < kSlices) {
      p = partials[(i * kSlices + threadIdx.x) * 2];
      q = partials[(i * kSlices + threadIdx.x) * 2 + 1];
    }
    block_sum2(p, q, sh);
    if (threadIdx.x == 0) terms[i] = r[i] * p + (1.0f - r[i]) * q;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float s = 0.0f;
    for (int64_t i = 0; i < n; ++i) s += terms[i];
    *loss = s / (float)n;
  }
}

}  // namespace

hipError_t launch_nft_noise(const float* x0, const float* eps, const float* t, int64_t n, int64_t d, float* xt,
                            hipStream_t st) {
  const int64_t d4 = d / 4;
  nft_noise_kernel<<<dim3(kSlices, (unsigned)n), kThreads, 0, st>>>(reinterpret_cast<const float4*>(x0),
                                                                   reinterpret_cast<const float4*>(eps), t, d4,
                                                                   reinterpret_cast<float4*>(xt));
  return hipGetLastError();
}

hipError_t launch_nft_loss(const float* v_old, const float* v_theta, const float* x0, const float* eps,
                           const float* r, float beta, int64_t n, int64_t d, float* partials, float* terms,
                           float* loss, hipStream_t st) {
  const int64_t d4 = d / 4;
  nft_loss_partial_kernel<<<dim3(kSlices, (unsigned)n), kThreads, 0, st>>>(
      reinterpret_cast<const float4*>(v_old), reinterpret_cast<const float4*>(v_theta),
      reinterpret_cast<const float4*>(x0), reinterpret_cast<const float4*>(eps), beta, d4, partials);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  nft_loss_final_kernel<<<1, kThreads, 0, st>>>(partials, r, n, terms, loss);
  return hipGetLastError();
}

}  // namespace fp4r
