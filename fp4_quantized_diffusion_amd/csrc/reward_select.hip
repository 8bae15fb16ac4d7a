// Proxy reward, reward normalisation and top/bottom seed selection for gfx950.
//
// Stage 1 of the Sol-RL pipeline scores its N candidates with a proxy reward
// and keeps the K/2 best and K/2 worst seeds (project page, "Two-Stage
// Pipeline"; aitrends summary, Stage-1 paragraph). The normalised reward is
// r = 1/2 + 1/2 clip((x - mean)/std, -1, 1) (VeRL-Omni DiffusionNFT docs,
// "Algorithm", first equation).
//
// Every reduction runs in a fixed order (no atomics), so results are
// bitwise repeatable.
#include "common.h"

namespace fp4r {
namespace {

constexpr int kRewardThreads = 1024;
constexpr int kRankThreads = 256;
constexpr int kRankChunk = 4096;

// One workgroup per candidate; the candidate's rows_per_cand x dim block is
// read once as float4 columns. u == NULL gives the plain mean.
__global__ __launch_bounds__(kRewardThreads) void proxy_reward_kernel(
    const float* __restrict__ x, int64_t rows, int64_t dim, int64_t ldx, const float* __restrict__ u,
    float* __restrict__ rewards) {
  __shared__ float sh[kRewardThreads / 64];
  const int64_t c = blockIdx.x;
  const int64_t d4 = dim >> 2;
  const int64_t total = rows * d4;
  const float* base = x + c * rows * ldx;
  float acc = 0.f;
  for (int64_t i = threadIdx.x; i < total; i += kRewardThreads) {
    const int64_t r = i / d4, q = i - r * d4;
    const float4 a = *reinterpret_cast<const float4*>(base + r * ldx + q * 4);
    if (u) {
      const float4 w = reinterpret_cast<const float4*>(u)[q];
      acc += a.x * w.x + a.y * w.y + a.z * w.z + a.w * w.w;
    } else {
      acc += (a.x + a.y) + (a.z + a.w);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < kRewardThreads / 64; ++w) t += sh[w];
    rewards[c] = u ? t / (float)rows : t / ((float)rows * (float)dim);
  }
}

// Position of each candidate in the total order (reward descending, ties by
// ascending index), by counting; positions < k_top go to top, positions
// >= n - k_bottom go to bottom (lowest first).
__global__ __launch_bounds__(kRankThreads) void rank_kernel(const float* __restrict__ r, int n, int k_top,
                                                            int k_bottom, int32_t* __restrict__ top,
                                                            int32_t* __restrict__ bottom) {
  __shared__ float sr[kRankChunk];
  const int i = blockIdx.x * kRankThreads + threadIdx.x;
  const float ri = i < n ? r[i] : 0.f;
  int pos = 0;
  for (int base = 0; base < n; base += kRankChunk) {
    const int len = min(kRankChunk, n - base);
    __syncthreads();
    for (int j = threadIdx.x; j < len; j += kRankThreads) sr[j] = r[base + j];
    __syncthreads();
    if (i < n) {
      for (int j = 0; j < len; ++j) {
        const float rj = sr[j];
        pos += (rj > ri) || (rj == ri && base + j < i);
      }
    }
  }
  if (i < n) {
    if (pos < k_top) top[pos] = i;
    if (pos >= n - k_bottom) bottom[n - 1 - pos] = i;
  }
}

// Batch mean and population std in fp64 (fixed order), then r_norm.
__global__ __launch_bounds__(kRankThreads) void normalize_kernel(const float* __restrict__ r, int n,
                                                                 float* __restrict__ r_norm) {
  __shared__ double sh[kRankThreads];
  double s = 0.0;
  for (int j = threadIdx.x; j < n; j += kRankThreads) s += (double)r[j];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int o = kRankThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  const double mu = sh[0] / (double)n;
  __syncthreads();
  double q = 0.0;
  for (int j = threadIdx.x; j < n; j += kRankThreads) {
    const double d = (double)r[j] - mu;
    q += d * d;
  }
  sh[threadIdx.x] = q;
  __syncthreads();
  for (int o = kRankThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  const double sd = sqrt(sh[0] / (double)n);
  for (int j = threadIdx.x; j < n; j += kRankThreads) {
    double z = sd == 0.0 ? 0.0 : ((double)r[j] - mu) / sd;
    z = z < -1.0 ? -1.0 : (z > 1.0 ? 1.0 : z);
    r_norm[j] = (float)(0.5 + 0.5 * z);
  }
}

}  // namespace

hipError_t launch_proxy_reward(const float* x, int64_t n_cand, int64_t rows_per_cand, int64_t dim,
                               int64_t ldx, const float* u, float* rewards, hipStream_t st) {
  proxy_reward_kernel<<<(unsigned)n_cand, kRewardThreads, 0, st>>>(x, rows_per_cand, dim, ldx, u, rewards);
  return hipGetLastError();
}

hipError_t launch_select(const float* r, int64_t n, int64_t k_top, int64_t k_bottom, int32_t* top,
                         int32_t* bottom, float* r_norm, hipStream_t st) {
  const unsigned g = (unsigned)((n + kRankThreads - 1) / kRankThreads);
  rank_kernel<<<g, kRankThreads, 0, st>>>(r, (int)n, (int)k_top, (int)k_bottom, top, bottom);
  if (r_norm) normalize_kernel<<<1, kRankThreads, 0, st>>>(r, (int)n, r_norm);
  return hipGetLastError();
}

}  // namespace fp4r
