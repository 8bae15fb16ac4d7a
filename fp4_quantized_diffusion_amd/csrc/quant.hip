// Block-scaled 4-bit quantization kernels (MXFP4 and NVFP4-style) for gfx950.
//
// The rollout re-quantizes its weights every iteration and quantizes the
// activations entering every solver linear (Sol-RL project page, "Two-Stage
// Pipeline"). Both are HBM-bound streams: the kernels read each input element
// once (RMSNorm rows longer than 4096 elements twice, the second time from
// L2), write half a byte of code per element and one scale byte per block,
// and keep every decision in integer or exactly-rounded fp32 arithmetic so
// the codes are bit-identical to the format's definition.
//
// Thread layout: every thread owns 8 consecutive elements of one row
// ("octet"); the 4 (MX, block 32) or 2 (NV, block 16) threads of a block are
// adjacent lanes and combine their block maximum with lane shuffles. Input
// reads are 16-byte vector loads, code writes one 32-bit store per thread.
// This file is compiled with -ffp-contract=off: every fp32 operation below
// rounds on its own.
#include "quant_common.h"

namespace fp4r {
namespace {

constexpr int kThreads = 256;

// Store of codes and scales, which are written once and read by a later
// kernel: non-temporal (NT) where that measured faster -- the plain
// quantizers (MX: 2.37 -> 2.24 ms for 393216 x 12288 bf16) -- and ordinary
// for the fused GELU and RMSNorm prologues, which NT stores slowed down
// (2.82 -> 3.01 ms and 1.16 -> 1.29 ms).
template <bool NT, class T>
__device__ __forceinline__ void st_out(T* p, T v) {
  if (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

enum { PRO_NONE = 0, PRO_RMSNORM = 1, PRO_GELU = 2 };

// Elementwise prologue of one loaded octet (tab: the GELU table -- of Q at
// every bf16 magnitude for bf16 input, of (Q, phi) for fp32 input).
template <int BF16, int PRO>
__device__ __forceinline__ void prologue8(float v[8], const void* tab) {
  if (PRO == PRO_GELU) {
    if (BF16) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = gelu_bf16(v[j], static_cast<const float*>(tab));
    } else {
      float z[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) z[j] = v[j];
      gelu_f32_tab_n<8>(v, z, static_cast<const float2*>(tab));
    }
  }
}

// LDS for the GELU table when the kernel needs it (GELU prologue).
template <int BF16, int PRO>
struct GeluLds {
  __device__ __forceinline__ const void* get() { return nullptr; }
};
template <>
struct GeluLds<1, PRO_GELU> {
  __device__ __forceinline__ const void* get() {
    __shared__ float tab[kGeluTab];
    gelu_table_fill(tab);
    __syncthreads();
    return tab;
  }
};
template <>
struct GeluLds<0, PRO_GELU> {
  __device__ __forceinline__ const void* get() {
    __shared__ float2 tab[kGeluTTab];
    gelu_table_fill(tab);
    __syncthreads();
    return tab;
  }
};

// Steps a thread works on at once in the elementwise kernels: their loads
// are all issued before the first is used, so each wave keeps four 16-byte
// loads per lane in flight.
constexpr int kUnroll = 4;
// The NVFP4-style passes keep two steps in flight: with four they took 2-3%
// longer (the code pass carries more registers per step), with eight 5-8%.
constexpr int kUnrollNv = 2;

// n / d for a workgroup-uniform step index n and a divisor fixed per launch,
// without a 64-bit division in the loop: one high multiply, an add and two
// shifts (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994, the unsigned N = 32 case: l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1, q = (t + ((n - t) >> min(l, 1))) >>
// max(l - 1, 0) with t the high word of m n), exact for every n < 2^32.
// Larger n (or d) take the plain division.
struct UDiv {
  int64_t d, lim;  // lim: 2^32 when d < 2^32, else 0 (fast path off)
  uint32_t m, s1, s2;
};

UDiv make_udiv(int64_t d) {  // d >= 1
  UDiv f{d, 0, 0u, 0u, 0u};
  if (d >= ((int64_t)1 << 32)) return f;
  int l = 0;
  while (((int64_t)1 << l) < d) ++l;
  f.lim = (int64_t)1 << 32;
  f.m = (uint32_t)(((((uint64_t)1 << l) - (uint64_t)d) << 32) / (uint64_t)d + 1u);
  f.s1 = l < 1 ? (uint32_t)l : 1u;
  f.s2 = l > 1 ? (uint32_t)(l - 1) : 0u;
  return f;
}

__device__ __forceinline__ int64_t udiv(int64_t n, const UDiv& f) {
  if (n < f.lim) {
    const uint32_t x = (uint32_t)n, t = __umulhi(x, f.m);
    return (int64_t)((t + ((x - t) >> f.s1)) >> f.s2);
  }
  return n / f.d;
}

// Row-major layout, elementwise prologues. Work comes in steps of 256
// consecutive octets of one row (segs steps per row); a step's row and
// segment are workgroup-uniform, so the index arithmetic is scalar.
template <int BF16, int PRO>
__global__ __launch_bounds__(kThreads) void quant_mx_kernel(
    const void* __restrict__ x, int64_t ldx, uint8_t* __restrict__ codes, int64_t ld_codes,
    uint8_t* __restrict__ scales, int64_t ld_scales, int64_t opr, UDiv segs, int64_t steps) {
  const void* tab = GeluLds<BF16, PRO>().get();
  const int64_t G = gridDim.x;
  for (int64_t st0 = blockIdx.x; st0 < steps; st0 += kUnroll * G) {
    float v[kUnroll][8];
    int64_t row[kUnroll], oct[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t st = st0 + u * G;
      row[u] = udiv(st, segs);
      oct[u] = (st - row[u] * segs.d) * kThreads + threadIdx.x;
      // unconditional loads (an idle lane reads the first octet), so that
      // all of them are in flight before the first is waited for
      const bool ok = st < steps && oct[u] < opr;
      load8<BF16>(x, ok ? row[u] * ldx + oct[u] * 8 : 0, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // whole 32-blocks drop out: opr is a multiple of 4
      if (st0 + u * G >= steps || oct[u] >= opr) continue;
      prologue8<BF16, PRO>(v[u], tab);
      uint32_t S;
      const uint32_t w = mx_block(v[u], S);
      st_out<PRO == PRO_NONE>(reinterpret_cast<uint32_t*>(codes + row[u] * ld_codes + oct[u] * 4), w);
      if ((oct[u] & 3) == 0) st_out<PRO == PRO_NONE>(scales + row[u] * ld_scales + (oct[u] >> 2), (uint8_t)S);
    }
  }
}

// Panel layout: (panel of 256 rows, chunk of 128 elements) blocks of 256 x 16
// octets; octet i (= step * 256 + thread) is octet i % 16 of row i / 16 % 256
// in block i / 4096, so its code word lands at byte 4 i and its block's scale
// byte at i / 4 -- every wave writes 256 contiguous code bytes. A step lies
// in one block, so panel and chunk are workgroup-uniform. Rows past `rows`
// and elements past k are padding: code 0, scale byte 127.
template <int BF16, int PRO>
__global__ __launch_bounds__(kThreads) void quant_mx_panel_kernel(
    const void* __restrict__ x, int64_t rows, int64_t k, int64_t ldx, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, UDiv nc, int64_t steps) {
  const void* tab = GeluLds<BF16, PRO>().get();
  const int64_t G = gridDim.x;
  for (int64_t st0 = blockIdx.x; st0 < steps; st0 += kUnroll * G) {
    float v[kUnroll][8];
    bool valid[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t st = st0 + u * G;
      const int64_t blk = st >> 4;
      const int64_t pnl = udiv(blk, nc), ch = blk - pnl * nc.d;
      const int64_t row = pnl * 256 + (int)((st & 15) << 4) + (int)(threadIdx.x >> 4);
      const int64_t e0 = ch * 128 + (int)(threadIdx.x & 15) * 8;
      // a 32-block's 4 octets share row and validity (k is a multiple of 32)
      valid[u] = st < steps && row < rows && e0 < k;
      // unconditional loads (an idle lane reads the first octet), so that
      // all of them are in flight before the first is waited for
      load8<BF16>(x, valid[u] ? row * ldx + e0 : 0, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t st = st0 + u * G;
      if (st >= steps) continue;  // workgroup-uniform
      prologue8<BF16, PRO>(v[u], tab);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[u][j] = valid[u] ? v[u][j] : 0.f;
      uint32_t S;
      const uint32_t w = mx_block(v[u], S);
      const int64_t i = st * kThreads + threadIdx.x;
      st_out<PRO == PRO_NONE>(reinterpret_cast<uint32_t*>(codes) + i, valid[u] ? w : 0u);
      if ((threadIdx.x & 3) == 0) st_out<PRO == PRO_NONE>(scales + (i >> 2), (uint8_t)(valid[u] ? S : 127u));
    }
  }
}

// Deterministic block-wide fp32 sum (fixed shuffle tree, then fixed LDS order).
__device__ float block_sum(float v, float* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  float t = 0.f;
  if (threadIdx.x == 0) {
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += sh[w];
    sh[8] = t;
  }
  __syncthreads();
  t = sh[8];
  __syncthreads();
  return t;
}

// RMSNorm prologue for rows of more than 4096 elements: one workgroup per
// row. Pass 1 sums squares, pass 2 normalizes (y = x * (1 / sqrt(mean +
// 1e-6)), unit gain) and quantizes.
template <int BF16>
__global__ __launch_bounds__(kThreads) void quant_mx_rmsnorm_kernel(
    const void* __restrict__ x, int64_t k, int64_t ldx, uint8_t* __restrict__ codes, int64_t ld_codes,
    uint8_t* __restrict__ scales, int64_t ld_scales) {
  __shared__ float sh[16];
  const int64_t row = blockIdx.x;
  const int64_t oct_per_row = k >> 3;
  float ss = 0.f;
  for (int64_t oct = threadIdx.x; oct < oct_per_row; oct += kThreads) {
    float v[8];
    load8<BF16>(x, row * ldx + oct * 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
  }
  const float tot = block_sum(ss, sh);
  const float inv = 1.0f / sqrtf(tot / (float)k + 1e-6f);
  for (int64_t oct = threadIdx.x; oct < oct_per_row; oct += kThreads) {
    float v[8];
    load8<BF16>(x, row * ldx + oct * 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] * inv;
    uint32_t am = amax_bits8(v);
    am = max(am, (uint32_t)__shfl_xor((int)am, 1));
    am = max(am, (uint32_t)__shfl_xor((int)am, 2));
    const uint32_t S = mx_scale(am);
    *reinterpret_cast<uint32_t*>(codes + row * ld_codes + oct * 4) = mx_pack8(v, S);
    if ((oct & 3) == 0) scales[row * ld_scales + (oct >> 2)] = (uint8_t)S;
  }
}

// RMSNorm prologue into the panel layout: one workgroup per row of the padded
// row range (rows past `rows` write padding only); same arithmetic as above.
template <int BF16>
__global__ __launch_bounds__(kThreads) void quant_mx_rmsnorm_panel_kernel(
    const void* __restrict__ x, int64_t rows, int64_t k, int64_t ldx, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t nc) {
  __shared__ float sh[16];
  const int64_t row = blockIdx.x;
  const bool row_valid = row < rows;  // uniform over the workgroup
  const int64_t oct_per_row = k >> 3;
  float ss = 0.f;
  if (row_valid) {
    for (int64_t oct = threadIdx.x; oct < oct_per_row; oct += kThreads) {
      float v[8];
      load8<BF16>(x, row * ldx + oct * 8, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
    }
  }
  const float tot = block_sum(ss, sh);
  const float inv = 1.0f / sqrtf(tot / (float)k + 1e-6f);
  const int64_t pnl = row >> 8, rr = row & 255;
  for (int64_t oct = threadIdx.x; oct < nc * 16; oct += kThreads) {
    const bool valid = row_valid && oct < oct_per_row;  // shared by a 32-block's 4 octets
    float v[8];
    if (valid) {
      load8<BF16>(x, row * ldx + oct * 8, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v[j] * inv;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.f;
    }
    uint32_t am = amax_bits8(v);
    am = max(am, (uint32_t)__shfl_xor((int)am, 1));
    am = max(am, (uint32_t)__shfl_xor((int)am, 2));
    const uint32_t S = mx_scale(am);
    const int64_t blk = pnl * nc + (oct >> 4);
    *reinterpret_cast<uint32_t*>(codes + (blk * 256 + rr) * 64 + (oct & 15) * 4) = valid ? mx_pack8(v, S) : 0u;
    if ((oct & 3) == 0) scales[(blk * 256 + rr) * 4 + ((oct & 15) >> 2)] = (uint8_t)(valid ? S : 127u);
  }
}

// Rows per workgroup of the register-resident RMSNorm quantizer: 16 (one
// per wave). Measured on 393216 x 3072 fp32 in the panel layout: 1099 us
// with 4 rows per workgroup, 1072 us with 8, 1059-1066 us with 16 (with
// non-temporal code stores, themselves worth about 1%); 1 row per
// workgroup took 1166 us.
constexpr int kRmsThreads = 1024;

// RMSNorm prologue with the row in registers: one wave per row (16 rows per
// workgroup), lane l holding octets l, l + 64, ..., l + 64 (NO - 1), so
// the row is read once and no workgroup-wide synchronization is needed. The
// sum of squares runs over the lane's octets in order, then over a fixed
// xor-shuffle tree (fp32 addition commutes, so every lane ends with the same
// total). The row-major and panel layouts run this same arithmetic, for any
// K with ceil(K / 512) <= 8 in both (K <= 4096); larger K takes the two-pass
// kernels above in both layouts. Octets past K (panel padding) hold zeros,
// which add nothing to the sum. PANEL: rows past `rows` up to the panel edge
// (nrows) write padding only.
template <int BF16, int NO, bool PANEL>
__global__ __launch_bounds__(kRmsThreads) void quant_mx_rmsnorm_wave_kernel(
    const void* __restrict__ x, int64_t rows, int64_t nrows, int64_t k, int64_t ldx, uint8_t* __restrict__ codes,
    int64_t ld_codes, uint8_t* __restrict__ scales, int64_t ld_scales, int64_t nc) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kRmsThreads / 64) + (threadIdx.x >> 6);
  if (row >= nrows) return;  // uniform over the wave
  const bool row_valid = row < rows;
  const int opr = (int)(k >> 3);
  float v[NO][8];
#pragma unroll
  for (int t = 0; t < NO; ++t) {
    const int o = lane + 64 * t;
    if (row_valid && o < opr) {
      load8<BF16>(x, row * ldx + (int64_t)o * 8, v[t]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[t][j] = 0.f;
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int t = 0; t < NO; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += v[t][j] * v[t][j];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv = 1.0f / sqrtf(ss / (float)k + 1e-6f);
  const int64_t pnl = row >> 8, rr = row & 255;
#pragma unroll
  for (int t = 0; t < NO; ++t) {
    const int o = lane + 64 * t;
    const bool valid = row_valid && o < opr;  // shared by a 32-block's 4 octets
#pragma unroll
    for (int j = 0; j < 8; ++j) v[t][j] = v[t][j] * inv;
    uint32_t S;
    const uint32_t w = mx_block(v[t], S);
    if (PANEL) {
      if (o < nc * 16) {
        const int64_t blk = pnl * nc + (o >> 4);
        __builtin_nontemporal_store(valid ? w : 0u, reinterpret_cast<uint32_t*>(codes + (blk * 256 + rr) * 64 + (o & 15) * 4));
        if ((o & 3) == 0) scales[(blk * 256 + rr) * 4 + ((o & 15) >> 2)] = (uint8_t)(valid ? S : 127u);
      }
    } else if (valid) {
      *reinterpret_cast<uint32_t*>(codes + row * ld_codes + (int64_t)o * 4) = w;
      if ((o & 3) == 0) scales[row * ld_scales + (o >> 2)] = (uint8_t)S;
    }
  }
}

// Launch the register-resident RMSNorm quantizer when the row fits (NO <= 8
// octets per lane); false otherwise.
template <int BF16, bool PANEL, int NO = 1>
void launch_rmsnorm_wave_no(int64_t no, unsigned g, const void* x, int64_t rows, int64_t nrows, int64_t k,
                            int64_t ldx, uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                            int64_t nc, hipStream_t st) {
  if constexpr (NO < 8) {
    if (no > NO) {
      launch_rmsnorm_wave_no<BF16, PANEL, NO + 1>(no, g, x, rows, nrows, k, ldx, codes, ld_codes, scales, ld_scales,
                                                  nc, st);
      return;
    }
  }
  quant_mx_rmsnorm_wave_kernel<BF16, NO, PANEL>
      <<<g, kRmsThreads, 0, st>>>(x, rows, nrows, k, ldx, codes, ld_codes, scales, ld_scales, nc);
}

template <bool PANEL>
bool launch_rmsnorm_wave(const void* x, int x_bf16, int64_t rows, int64_t nrows, int64_t k, int64_t ldx,
                         uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, int64_t nc,
                         hipStream_t st) {
  const int64_t octs = PANEL ? nc * 16 : (k >> 3);
  const int64_t no = (octs + 63) / 64;
  if (no < 1 || no > 8) return false;
  const unsigned g = (unsigned)((nrows + kRmsThreads / 64 - 1) / (kRmsThreads / 64));
  if (x_bf16)
    launch_rmsnorm_wave_no<1, PANEL>(no, g, x, rows, nrows, k, ldx, codes, ld_codes, scales, ld_scales, nc, st);
  else
    launch_rmsnorm_wave_no<0, PANEL>(no, g, x, rows, nrows, k, ldx, codes, ld_codes, scales, ld_scales, nc, st);
  return true;
}

// ---------------------------- NVFP4-style ----------------------------------

__global__ void nv_zero_kernel(float* ts) { *reinterpret_cast<uint32_t*>(ts) = 0u; }

// Tensor amax: |x| bit patterns order like the values, so an integer max is
// exact and order-independent (deterministic). Work comes in the row-major
// kernels' steps (256 consecutive octets of one row, workgroup-uniform row
// and segment), kUnrollNv steps per pass with all loads issued first.
template <int BF16>
__global__ __launch_bounds__(kThreads) void nv_amax_kernel(const void* __restrict__ x, int64_t ldx, int64_t opr,
                                                           UDiv segs, int64_t steps, float* ts) {
  __shared__ uint32_t sh[kThreads / 64];
  const int64_t G = gridDim.x;
  uint32_t m = 0;
  for (int64_t st0 = blockIdx.x; st0 < steps; st0 += kUnrollNv * G) {
    float v[kUnrollNv][8];
    bool ok[kUnrollNv];
#pragma unroll
    for (int u = 0; u < kUnrollNv; ++u) {
      const int64_t st = st0 + u * G;
      const int64_t row = udiv(st, segs);
      const int64_t oct = (st - row * segs.d) * kThreads + threadIdx.x;
      ok[u] = st < steps && oct < opr;
      load8<BF16>(x, ok[u] ? row * ldx + oct * 8 : 0, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnrollNv; ++u)
      if (ok[u]) m = max(m, amax_bits8(v[u]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kThreads / 64; ++w) t = max(t, sh[w]);
    amax_raise(ts, t);
  }
}

// s_g = fl(A_t / 2688); 1 where that quotient is 0 (all-zero tensor, or one
// so small the quotient underflows: its codes are signed zeros either way).
__global__ void nv_finalize_kernel(float* ts) {
  const float at = __uint_as_float(*reinterpret_cast<const uint32_t*>(ts));
  const float sg = at / 2688.0f;
  *ts = (sg == 0.0f) ? 1.0f : sg;
}

// Per-group tensor amax (GROUPED quantization: one tensor scale per group of
// rpg rows, e.g. per candidate): workgroup (g, s) takes slice s of group g's
// rows, one integer atomicMax at its end, as nv_amax_kernel.
template <int BF16>
__global__ __launch_bounds__(kThreads) void nv_amax_group_kernel(const void* __restrict__ x, int64_t ldx, int64_t opr,
                                                                 int64_t rpg, int64_t rows_per_slice, float* ts) {
  __shared__ uint32_t sh[kThreads / 64];
  const int64_t g = blockIdx.x;
  const int64_t r0 = g * rpg + (int64_t)blockIdx.y * rows_per_slice;
  const int64_t r1 = min(r0 + rows_per_slice, (g + 1) * rpg);
  uint32_t m = 0;
  for (int64_t row = r0; row < r1; ++row)
    for (int64_t oct = threadIdx.x; oct < opr; oct += kThreads) {
      float v[8];
      load8<BF16>(x, row * ldx + oct * 8, v);
      m = max(m, amax_bits8(v));
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kThreads / 64; ++w) t = max(t, sh[w]);
    amax_raise(ts + g, t);
  }
}

__global__ void nv_zero_groups_kernel(float* ts, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) reinterpret_cast<uint32_t*>(ts)[i] = 0u;
}

// s_g of every group, as nv_finalize_kernel.
__global__ void nv_finalize_groups_kernel(float* ts, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float at = __uint_as_float(reinterpret_cast<const uint32_t*>(ts)[i]);
  const float sg = at / 2688.0f;
  ts[i] = (sg == 0.0f) ? 1.0f : sg;
}

// Codes and E4M3 block scales, in the row-major kernels' steps (a 16-block is
// two adjacent lanes of one step), kUnrollNv steps per pass. GROUPED: the
// tensor scale of row r is ts[r / rpg].
template <int BF16, bool GROUPED>
__global__ __launch_bounds__(kThreads) void quant_nv_kernel(
    const void* __restrict__ x, int64_t ldx, uint8_t* __restrict__ codes, int64_t ld_codes,
    uint8_t* __restrict__ scales, int64_t ld_scales, int64_t opr, UDiv segs, int64_t steps,
    const float* __restrict__ ts, UDiv rpg) {
  const float sg0 = GROUPED ? 0.0f : *ts;
  const float tau0 = 6.0f * sg0;
  const int64_t G = gridDim.x;
  for (int64_t st0 = blockIdx.x; st0 < steps; st0 += kUnrollNv * G) {
    float vv[kUnrollNv][8];
    int64_t rows[kUnrollNv], octs[kUnrollNv];
#pragma unroll
    for (int u = 0; u < kUnrollNv; ++u) {
      const int64_t st = st0 + u * G;
      rows[u] = udiv(st, segs);
      octs[u] = (st - rows[u] * segs.d) * kThreads + threadIdx.x;
      const bool ok = st < steps && octs[u] < opr;
      load8<BF16>(x, ok ? rows[u] * ldx + octs[u] * 8 : 0, vv[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnrollNv; ++u) {
    // whole 16-blocks drop out: opr is even
    if (st0 + u * G >= steps || octs[u] >= opr) continue;
    const int64_t row = rows[u], oct = octs[u];
    const float sg = GROUPED ? ts[udiv(row, rpg)] : sg0;  // row is uniform over the workgroup
    const float tau = GROUPED ? 6.0f * sg : tau0;
    uint32_t S;
    const uint32_t w = nv_block(vv[u], sg, tau, S);
    st_out<true>(reinterpret_cast<uint32_t*>(codes + row * ld_codes + oct * 4), w);
    if ((oct & 1) == 0) st_out<true>(scales + row * ld_scales + (oct >> 1), (uint8_t)S);
    }
  }
}

inline unsigned grid_for(int64_t work_items) {
  int64_t g = (work_items + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  if (g > (1 << 20)) g = 1 << 20;
  return (unsigned)g;
}

// Grid of an elementwise kernel over `steps` workgroup steps, kUnroll per
// workgroup pass. A kernel that first fills an LDS table is instead given
// exactly as many workgroups as fit on the GPU at once (each then walks its
// share of the steps), so the table is filled once per resident workgroup.
template <class Kernel>
unsigned elementwise_grid(Kernel kernel, int64_t steps, bool table) {
  unsigned g = grid_for((steps + kUnroll - 1) / kUnroll * kThreads);
  if (!table) return g;
  // per kernel instantiation, queried once (thread-safe static
  // initialization) on the device current at the first call; the library
  // runs on one kind of GPU
  static const int resident = [kernel] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess || cus <= 0 ||
        per_cu <= 0)
      return 1024;
    return cus * per_cu;
  }();
  return g < (unsigned)resident ? g : (unsigned)resident;
}

}  // namespace

hipError_t launch_quant_mx(const void* x, int x_bf16, int64_t rows, int64_t k, int64_t ldx,
                           uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                           int prologue, hipStream_t st) {
  if (prologue == PRO_RMSNORM) {
    if (launch_rmsnorm_wave<false>(x, x_bf16, rows, rows, k, ldx, codes, ld_codes, scales, ld_scales, 0, st))
      return hipGetLastError();
    if (x_bf16)
      quant_mx_rmsnorm_kernel<1><<<(unsigned)rows, kThreads, 0, st>>>(x, k, ldx, codes, ld_codes, scales, ld_scales);
    else
      quant_mx_rmsnorm_kernel<0><<<(unsigned)rows, kThreads, 0, st>>>(x, k, ldx, codes, ld_codes, scales, ld_scales);
    return hipGetLastError();
  }
  const int64_t opr = k >> 3, segs = (opr + kThreads - 1) / kThreads, steps = rows * segs;
#define FP4R_LAUNCH(B, P, TAB)                                                                             \
  quant_mx_kernel<B, P><<<elementwise_grid(quant_mx_kernel<B, P>, steps, TAB), kThreads, 0, st>>>(         \
      x, ldx, codes, ld_codes, scales, ld_scales, opr, make_udiv(segs), steps)
  if (prologue == PRO_GELU) {
    if (x_bf16) FP4R_LAUNCH(1, PRO_GELU, true);
    else FP4R_LAUNCH(0, PRO_GELU, true);
  } else {
    if (x_bf16) FP4R_LAUNCH(1, PRO_NONE, false);
    else FP4R_LAUNCH(0, PRO_NONE, false);
  }
#undef FP4R_LAUNCH
  return hipGetLastError();
}

hipError_t launch_quant_mx_panel(const void* x, int x_bf16, int64_t rows, int64_t k, int64_t ldx, uint8_t* codes,
                                 uint8_t* scales, int prologue, hipStream_t st) {
  const int64_t panels = (rows + 255) >> 8, nc = (k + 127) >> 7;
  if (prologue == PRO_RMSNORM) {
    if (launch_rmsnorm_wave<true>(x, x_bf16, rows, panels * 256, k, ldx, codes, 0, scales, 0, nc, st))
      return hipGetLastError();
    const unsigned g = (unsigned)(panels * 256);
    if (x_bf16)
      quant_mx_rmsnorm_panel_kernel<1><<<g, kThreads, 0, st>>>(x, rows, k, ldx, codes, scales, nc);
    else
      quant_mx_rmsnorm_panel_kernel<0><<<g, kThreads, 0, st>>>(x, rows, k, ldx, codes, scales, nc);
    return hipGetLastError();
  }
  const int64_t steps = panels * nc * 16;  // 256 octets per step, 16 steps per (panel, chunk) block
#define FP4R_LAUNCH(B, P, TAB)                                                                             \
  quant_mx_panel_kernel<B, P><<<elementwise_grid(quant_mx_panel_kernel<B, P>, steps, TAB), kThreads, 0, st>>>( \
      x, rows, k, ldx, codes, scales, make_udiv(nc), steps)
  if (prologue == PRO_GELU) {
    if (x_bf16) FP4R_LAUNCH(1, PRO_GELU, true);
    else FP4R_LAUNCH(0, PRO_GELU, true);
  } else {
    if (x_bf16) FP4R_LAUNCH(1, PRO_NONE, false);
    else FP4R_LAUNCH(0, PRO_NONE, false);
  }
#undef FP4R_LAUNCH
  return hipGetLastError();
}

hipError_t launch_nv_scale_reset(float* ts, hipStream_t st) {
  nv_zero_kernel<<<1, 1, 0, st>>>(ts);
  return hipGetLastError();
}

hipError_t launch_nv_scale_finalize(float* ts, hipStream_t st) {
  nv_finalize_kernel<<<1, 1, 0, st>>>(ts);
  return hipGetLastError();
}

hipError_t launch_quant_nv(const void* x, int x_bf16, int64_t rows, int64_t k, int64_t ldx,
                           uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                           float* tensor_scale, int scale_given, hipStream_t st) {
  const int64_t opr = k >> 3, segs = (opr + kThreads - 1) / kThreads, steps = rows * segs;
  const unsigned g = grid_for((steps + kUnrollNv - 1) / kUnrollNv * kThreads);
  if (!scale_given) {
    nv_zero_kernel<<<1, 1, 0, st>>>(tensor_scale);
    // a resident-sized grid: each workgroup issues one atomic at its end
    const unsigned ga = g < 2048 ? g : 2048;
    if (x_bf16)
      nv_amax_kernel<1><<<ga, kThreads, 0, st>>>(x, ldx, opr, make_udiv(segs), steps, tensor_scale);
    else
      nv_amax_kernel<0><<<ga, kThreads, 0, st>>>(x, ldx, opr, make_udiv(segs), steps, tensor_scale);
    nv_finalize_kernel<<<1, 1, 0, st>>>(tensor_scale);
  }
  if (x_bf16)
    quant_nv_kernel<1, false><<<g, kThreads, 0, st>>>(x, ldx, codes, ld_codes, scales, ld_scales, opr,
                                                       make_udiv(segs), steps, tensor_scale, make_udiv(1));
  else
    quant_nv_kernel<0, false><<<g, kThreads, 0, st>>>(x, ldx, codes, ld_codes, scales, ld_scales, opr,
                                                       make_udiv(segs), steps, tensor_scale, make_udiv(1));
  return hipGetLastError();
}

hipError_t launch_quant_nv_grouped(const void* x, int x_bf16, int64_t rows, int64_t k, int64_t ldx, int64_t rpg,
                                   uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                                   float* tensor_scales, int scale_given, hipStream_t st) {
  const int64_t opr = k >> 3, segs = (opr + kThreads - 1) / kThreads, steps = rows * segs;
  const int64_t groups = rows / rpg;
  const unsigned g = grid_for((steps + kUnrollNv - 1) / kUnrollNv * kThreads);
  if (!scale_given) {
    const unsigned gz = (unsigned)((groups + 255) / 256);
    nv_zero_groups_kernel<<<gz, 256, 0, st>>>(tensor_scales, groups);
    // about 2048 workgroups in all: slices of each group's rows
    int64_t slices = (2048 + groups - 1) / groups;
    if (slices > rpg) slices = rpg;
    if (slices > 65535) slices = 65535;
    const int64_t rps = (rpg + slices - 1) / slices;
    slices = (rpg + rps - 1) / rps;
    const dim3 ga((unsigned)groups, (unsigned)slices);
    if (x_bf16)
      nv_amax_group_kernel<1><<<ga, kThreads, 0, st>>>(x, ldx, opr, rpg, rps, tensor_scales);
    else
      nv_amax_group_kernel<0><<<ga, kThreads, 0, st>>>(x, ldx, opr, rpg, rps, tensor_scales);
    nv_finalize_groups_kernel<<<gz, 256, 0, st>>>(tensor_scales, groups);
  }
  if (x_bf16)
    quant_nv_kernel<1, true><<<g, kThreads, 0, st>>>(x, ldx, codes, ld_codes, scales, ld_scales, opr,
                                                      make_udiv(segs), steps, tensor_scales, make_udiv(rpg));
  else
    quant_nv_kernel<0, true><<<g, kThreads, 0, st>>>(x, ldx, codes, ld_codes, scales, ld_scales, opr,
                                                      make_udiv(segs), steps, tensor_scales, make_udiv(rpg));
  return hipGetLastError();
}

}  // namespace fp4r
