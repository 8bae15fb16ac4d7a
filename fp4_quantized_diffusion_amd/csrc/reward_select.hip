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

// One workgroup per candidate, read once as float4 column groups: with
// dim % 4 == 0 and dim / 4 <= 1024 (the rollout's 3072 dims are 768 groups),
// thread t owns column group t for every row -- its weights u stay in
// registers, there is no index division, and each thread keeps kRows
// 16-byte loads in flight (256 KiB per workgroup: one workgroup per
// candidate leaves most CUs idle at 96 candidates, so each must keep many
// bytes in flight). Other shapes take the flat loop. u == NULL gives the
// plain mean. The sum runs in a fixed order (per thread over the rows in
// order, then a fixed shuffle tree and a fixed LDS order), so it is bitwise
// repeatable and independent of kRows.
constexpr int kRows = 16;

__device__ __forceinline__ float dot4(float4 a, float4 w) { return a.x * w.x + a.y * w.y + a.z * w.z + a.w * w.w; }

__global__ __launch_bounds__(kRewardThreads) void proxy_reward_kernel(
    const float* __restrict__ x, int64_t rows, int64_t dim, int64_t ldx, const float* __restrict__ u,
    float* __restrict__ rewards) {
  __shared__ float sh[kRewardThreads / 64];
  const int64_t c = blockIdx.x;
  const int64_t d4 = dim >> 2;
  const float* base = x + c * rows * ldx;
  float acc = 0.f;
  if ((dim & 3) == 0 && (ldx & 3) == 0 && d4 <= kRewardThreads) {
    const int t = threadIdx.x;
    if (t < d4) {
      const float4 w = u ? reinterpret_cast<const float4*>(u)[t] : make_float4(1.f, 1.f, 1.f, 1.f);
      const float* col = base + 4 * t;
      int64_t r = 0;
      for (; r + kRows <= rows; r += kRows) {
        float4 a[kRows];
#pragma unroll
        for (int j = 0; j < kRows; ++j) a[j] = *reinterpret_cast<const float4*>(col + (r + j) * ldx);
#pragma unroll
        for (int j = 0; j < kRows; ++j) acc += u ? dot4(a[j], w) : (a[j].x + a[j].y) + (a[j].z + a[j].w);
      }
      for (; r < rows; ++r) {
        const float4 a = *reinterpret_cast<const float4*>(col + r * ldx);
        acc += u ? dot4(a, w) : (a.x + a.y) + (a.z + a.w);
      }
    }
  } else {
    for (int64_t i = threadIdx.x; i < rows * dim; i += kRewardThreads) {
      const int64_t r = i / dim, q = i - r * dim;
      acc += u ? base[r * ldx + q] * u[q] : base[r * ldx + q];
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
// >= n - k_bottom go to bottom (lowest first). Rewards are compared through
// an integer key that orders every float: finite values and infinities by
// value (-0 and +0 equal), every NaN below -inf. The positions then form a
// permutation of 0..n-1 whatever the rewards hold, so every requested slot of
// top and bottom is written exactly once.
__device__ __forceinline__ uint32_t order_key(float v) {
  if (v != v) return 0u;                                         // NaN: below everything
  const uint32_t b = v == 0.0f ? 0u : __float_as_uint(v);        // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);             // -inf -> 0x007FFFFF
}

__global__ __launch_bounds__(kRankThreads) void rank_kernel(const float* __restrict__ r, int n, int k_top,
                                                            int k_bottom, int32_t* __restrict__ top,
                                                            int32_t* __restrict__ bottom) {
  __shared__ uint32_t sr[kRankChunk];
  const int i = blockIdx.x * kRankThreads + threadIdx.x;
  const uint32_t ki = i < n ? order_key(r[i]) : 0u;
  int pos = 0;
  for (int base = 0; base < n; base += kRankChunk) {
    const int len = min(kRankChunk, n - base);
    __syncthreads();
    for (int j = threadIdx.x; j < len; j += kRankThreads) sr[j] = order_key(r[base + j]);
    __syncthreads();
    if (i < n) {
      for (int j = 0; j < len; ++j) {
        const uint32_t kj = sr[j];
        pos += (kj > ki) || (kj == ki && base + j < i);
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
