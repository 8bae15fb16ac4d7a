// LoRA merge and re-quantization of a weight (MXFP4 or NVFP4-style), for
// gfx950.
//
// After each policy update the adapted weights are re-quantized at run time
// for the next FP4 rollout (Sol-RL project page, "Two-Stage Pipeline",
// Stage 2; aitrends summary, Stage-2 paragraph: LoRA of rank 32, real-time
// re-quantization with no compile step). With W [N, K] (nn.Linear layout),
// B [N, r] and A [r, K] the kernels form
//     acc = sum_j B[n, j] A[j, k]   (fp32 fma, j = 0 .. r-1 in order)
//     W'[n, k] = fma(s, acc, W[n, k])
// and quantize W' by the MX rule (one pass) or the NVFP4-style rule (a pass
// for the tensor amax of W', unless the tensor scale is given, then a pass
// that recomputes W' bit for bit and quantizes it), so the merged weight
// never goes to HBM.
//
// Work: one 256-thread workgroup per tile of 32 weight rows x 256 columns.
// The tile's slice of A ([r][256]) and rows of B ([32][r]) are staged in LDS
// as fp32; thread t owns column octet t % 32 of rows t / 32 + 8 i
// (i = 0..3), so an MX 32-block's 4 octets (an NV 16-block's 2) sit in
// adjacent lanes of one row.
// Per adapter index j a lane reads 8 values of A (two 16-byte LDS reads, the
// same addresses in both lane halves) and 4 of B (broadcasts), then does 32
// fmas. The W octets are loaded before the staging, so their latency hides
// behind it. Compiled with -ffp-contract=off; every fma is explicit.
#include "quant_common.h"

namespace fp4r {
namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 32;
constexpr int kRowsPerThread = kTileRows / (kThreads / 32);  // rows rg + 8 i of a thread
constexpr int kTileCols = 256;

template <int BF16>
__device__ __forceinline__ float load1(const void* p, int64_t i) {
  if (BF16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
  return reinterpret_cast<const float*>(p)[i];
}

// The merged values of one thread's 4 rows x 8 columns of the workgroup's
// tile: out[i][e] = fma(scale, acc, W) for row r0 + rg + 8 i and column
// 8 og + e, 0 where that element lies outside the weight (valid[i] false).
// Every thread of the workgroup must call it (it stages A and B in LDS
// behind a barrier).
template <int WBF16, int ABBF16>
__device__ __forceinline__ void lora_merge(const void* __restrict__ w, int64_t rows, int64_t k, int64_t ldw,
                                           const void* __restrict__ lb, int64_t ldb, const void* __restrict__ la,
                                           int64_t lda, int rank, float scale, float* lds, float out[kRowsPerThread][8],
                                           bool valid[kRowsPerThread]) {
  float* sa = lds;                        // [rank][kTileCols]
  float* sb = lds + rank * kTileCols;     // [kTileRows][rank]
  const int64_t r0 = (int64_t)blockIdx.y * kTileRows;
  const int64_t c0 = (int64_t)blockIdx.x * kTileCols;
  const int o = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int64_t og = (c0 >> 3) + o;            // global octet index along K
  const bool col_ok = og * 8 < k;              // shared by a block's octets (k % 16 == 0)

  float wv[kRowsPerThread][8];
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int64_t row = r0 + rg + 8 * i;
    valid[i] = row < rows && col_ok;
    if (valid[i]) {
      load8<WBF16>(w, row * ldw + og * 8, wv[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[i][e] = 0.f;
    }
  }
  for (int i = threadIdx.x; i < rank * kTileCols; i += kThreads) {
    const int j = i / kTileCols, c = i % kTileCols;
    sa[i] = c0 + c < k ? load1<ABBF16>(la, j * lda + c0 + c) : 0.f;
  }
  for (int i = threadIdx.x; i < kTileRows * rank; i += kThreads) {
    const int rr = i / rank, j = i - rr * rank;
    sb[i] = r0 + rr < rows ? load1<ABBF16>(lb, (r0 + rr) * ldb + j) : 0.f;
  }
  __syncthreads();

  float acc[kRowsPerThread][8];
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  for (int j = 0; j < rank; ++j) {
    const float4 a0 = *reinterpret_cast<const float4*>(sa + j * kTileCols + 8 * o);
    const float4 a1 = *reinterpret_cast<const float4*>(sa + j * kTileCols + 8 * o + 4);
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const float bv = sb[(rg + 8 * i) * rank + j];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(bv, av[e], acc[i][e]);
    }
  }
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) out[i][e] = valid[i] ? fmaf(scale, acc[i][e], wv[i][e]) : 0.f;
}

// MX. PANEL: the grid covers the padded extent (nrows = whole panels, nc =
// whole 128-element chunks) and writes zero codes with scale byte 127 there,
// as the panel quantizer does.
template <int WBF16, int ABBF16, bool PANEL>
__global__ __launch_bounds__(kThreads) void quant_mx_lora_kernel(
    const void* __restrict__ w, int64_t rows, int64_t k, int64_t ldw, const void* __restrict__ lb, int64_t ldb,
    const void* __restrict__ la, int64_t lda, int rank, float scale, uint8_t* __restrict__ codes, int64_t ld_codes,
    uint8_t* __restrict__ scales, int64_t ld_scales, int64_t nrows, int64_t nc) {
  extern __shared__ float lds[];
  float v[kRowsPerThread][8];
  bool valid[kRowsPerThread];
  lora_merge<WBF16, ABBF16>(w, rows, k, ldw, lb, ldb, la, lda, rank, scale, lds, v, valid);
  const int64_t r0 = (int64_t)blockIdx.y * kTileRows;
  const int o = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int64_t og = ((int64_t)blockIdx.x * kTileCols >> 3) + o;
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int64_t row = r0 + rg + 8 * i;  // the same for a 32-block's 4 lanes
    if (row >= nrows) continue;
    uint32_t S;
    const uint32_t wd = mx_block(v[i], S);
    if (PANEL) {
      if (og < nc * 16) {
        const int64_t blk = (row >> 8) * nc + (og >> 4), rr = row & 255;
        *reinterpret_cast<uint32_t*>(codes + (blk * 256 + rr) * 64 + (og & 15) * 4) = valid[i] ? wd : 0u;
        if ((og & 3) == 0) scales[(blk * 256 + rr) * 4 + ((og & 15) >> 2)] = (uint8_t)(valid[i] ? S : 127u);
      }
    } else if (valid[i]) {
      *reinterpret_cast<uint32_t*>(codes + row * ld_codes + og * 4) = wd;
      if ((og & 3) == 0) scales[row * ld_scales + (og >> 2)] = (uint8_t)S;
    }
  }
}

// NVFP4-style, pass 1 (no tensor scale given): max |W'| over the workgroup's
// tile into the amax word as an integer atomicMax on the float bits (exact
// and order-free for non-negative values).
template <int WBF16, int ABBF16>
__global__ __launch_bounds__(kThreads) void amax_nv_lora_kernel(
    const void* __restrict__ w, int64_t rows, int64_t k, int64_t ldw, const void* __restrict__ lb, int64_t ldb,
    const void* __restrict__ la, int64_t lda, int rank, float scale, float* ts) {
  extern __shared__ float lds[];
  __shared__ uint32_t sh[kThreads / 64];
  float v[kRowsPerThread][8];
  bool valid[kRowsPerThread];
  lora_merge<WBF16, ABBF16>(w, rows, k, ldw, lb, ldb, la, lda, rank, scale, lds, v, valid);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) m = max(m, amax_bits8(v[i]));  // outside elements are 0
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int wv = 0; wv < kThreads / 64; ++wv) t = max(t, sh[wv]);
    amax_raise(ts, t);
  }
}

// NVFP4-style, pass 2: the same merged values (recomputed, bit for bit),
// quantized with the tensor scale *ts, row-major codes and E4M3 scales.
template <int WBF16, int ABBF16>
__global__ __launch_bounds__(kThreads) void quant_nv_lora_kernel(
    const void* __restrict__ w, int64_t rows, int64_t k, int64_t ldw, const void* __restrict__ lb, int64_t ldb,
    const void* __restrict__ la, int64_t lda, int rank, float scale, const float* __restrict__ ts,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ scales, int64_t ld_scales) {
  extern __shared__ float lds[];
  float v[kRowsPerThread][8];
  bool valid[kRowsPerThread];
  lora_merge<WBF16, ABBF16>(w, rows, k, ldw, lb, ldb, la, lda, rank, scale, lds, v, valid);
  const float sg = *ts, tau = 6.0f * sg;
  const int64_t r0 = (int64_t)blockIdx.y * kTileRows;
  const int o = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int64_t og = ((int64_t)blockIdx.x * kTileCols >> 3) + o;
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    if (!valid[i]) continue;  // the same for a 16-block's 2 lanes
    const int64_t row = r0 + rg + 8 * i;
    uint32_t S;
    const uint32_t wd = nv_block(v[i], sg, tau, S);
    *reinterpret_cast<uint32_t*>(codes + row * ld_codes + og * 4) = wd;
    if ((og & 1) == 0) scales[row * ld_scales + (og >> 1)] = (uint8_t)S;
  }
}

// Dynamic LDS above the default 64 KiB limit (ranks above 56) must be
// granted per kernel.
template <class Kernel>
hipError_t allow_lds(Kernel kernel, size_t lds_bytes) {
  if (lds_bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
}

template <int WBF16, int ABBF16, bool PANEL>
hipError_t launch_lora(dim3 grid, size_t lds_bytes, const void* w, int64_t rows, int64_t k, int64_t ldw,
                       const void* lb, int64_t ldb, const void* la, int64_t lda, int rank, float scale,
                       uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, int64_t nrows, int64_t nc,
                       hipStream_t st) {
  auto kernel = quant_mx_lora_kernel<WBF16, ABBF16, PANEL>;
  const hipError_t e = allow_lds(kernel, lds_bytes);
  if (e != hipSuccess) return e;
  kernel<<<grid, kThreads, lds_bytes, st>>>(w, rows, k, ldw, lb, ldb, la, lda, rank, scale, codes, ld_codes, scales,
                                            ld_scales, nrows, nc);
  return hipGetLastError();
}

template <int WBF16, int ABBF16>
hipError_t launch_lora_layout(bool panel, dim3 grid, size_t lds_bytes, const void* w, int64_t rows, int64_t k,
                              int64_t ldw, const void* lb, int64_t ldb, const void* la, int64_t lda, int rank,
                              float scale, uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                              int64_t nrows, int64_t nc, hipStream_t st) {
  return panel ? launch_lora<WBF16, ABBF16, true>(grid, lds_bytes, w, rows, k, ldw, lb, ldb, la, lda, rank, scale,
                                                  codes, ld_codes, scales, ld_scales, nrows, nc, st)
               : launch_lora<WBF16, ABBF16, false>(grid, lds_bytes, w, rows, k, ldw, lb, ldb, la, lda, rank, scale,
                                                   codes, ld_codes, scales, ld_scales, nrows, nc, st);
}

template <int WBF16, int ABBF16>
hipError_t launch_nv_lora(dim3 grid, size_t lds_bytes, const void* w, int64_t rows, int64_t k, int64_t ldw,
                          const void* lb, int64_t ldb, const void* la, int64_t lda, int rank, float scale,
                          uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, float* ts,
                          bool scale_given, hipStream_t st) {
  hipError_t e;
  if (!scale_given) {
    if ((e = launch_nv_scale_reset(ts, st)) != hipSuccess) return e;
    auto amax = amax_nv_lora_kernel<WBF16, ABBF16>;
    if ((e = allow_lds(amax, lds_bytes)) != hipSuccess) return e;
    amax<<<grid, kThreads, lds_bytes, st>>>(w, rows, k, ldw, lb, ldb, la, lda, rank, scale, ts);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_nv_scale_finalize(ts, st)) != hipSuccess) return e;
  }
  auto quant = quant_nv_lora_kernel<WBF16, ABBF16>;
  if ((e = allow_lds(quant, lds_bytes)) != hipSuccess) return e;
  quant<<<grid, kThreads, lds_bytes, st>>>(w, rows, k, ldw, lb, ldb, la, lda, rank, scale, ts, codes, ld_codes,
                                           scales, ld_scales);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_mx_lora(const void* w, int w_bf16, int64_t rows, int64_t k, int64_t ldw, const void* lb,
                                int64_t ldb, const void* la, int64_t lda, int ab_bf16, int rank, float scale,
                                uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, int panel,
                                hipStream_t st) {
  const int64_t nc = (k + 127) / 128;
  const int64_t nrows = panel ? (rows + 255) / 256 * 256 : rows;
  const int64_t ncols = panel ? nc * 128 : k;
  const dim3 grid((unsigned)((ncols + kTileCols - 1) / kTileCols), (unsigned)((nrows + kTileRows - 1) / kTileRows));
  const size_t lds_bytes = (size_t)rank * (kTileCols + kTileRows) * sizeof(float);
  if (w_bf16)
    return ab_bf16 ? launch_lora_layout<1, 1>(panel, grid, lds_bytes, w, rows, k, ldw, lb, ldb, la, lda, rank, scale,
                                              codes, ld_codes, scales, ld_scales, nrows, nc, st)
                   : launch_lora_layout<1, 0>(panel, grid, lds_bytes, w, rows, k, ldw, lb, ldb, la, lda, rank, scale,
                                              codes, ld_codes, scales, ld_scales, nrows, nc, st);
  return ab_bf16 ? launch_lora_layout<0, 1>(panel, grid, lds_bytes, w, rows, k, ldw, lb, ldb, la, lda, rank, scale,
                                            codes, ld_codes, scales, ld_scales, nrows, nc, st)
                 : launch_lora_layout<0, 0>(panel, grid, lds_bytes, w, rows, k, ldw, lb, ldb, la, lda, rank, scale,
                                            codes, ld_codes, scales, ld_scales, nrows, nc, st);
}

hipError_t launch_quant_nv_lora(const void* w, int w_bf16, int64_t rows, int64_t k, int64_t ldw, const void* lb,
                                int64_t ldb, const void* la, int64_t lda, int ab_bf16, int rank, float scale,
                                uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, float* ts,
                                int scale_given, hipStream_t st) {
  const dim3 grid((unsigned)((k + kTileCols - 1) / kTileCols), (unsigned)((rows + kTileRows - 1) / kTileRows));
  const size_t lds_bytes = (size_t)rank * (kTileCols + kTileRows) * sizeof(float);
  const bool given = scale_given != 0;
  if (w_bf16)
    return ab_bf16 ? launch_nv_lora<1, 1>(grid, lds_bytes, w, rows, k, ldw, lb, ldb, la, lda, rank, scale, codes,
                                          ld_codes, scales, ld_scales, ts, given, st)
                   : launch_nv_lora<1, 0>(grid, lds_bytes, w, rows, k, ldw, lb, ldb, la, lda, rank, scale, codes,
                                          ld_codes, scales, ld_scales, ts, given, st);
  return ab_bf16 ? launch_nv_lora<0, 1>(grid, lds_bytes, w, rows, k, ldw, lb, ldb, la, lda, rank, scale, codes,
                                        ld_codes, scales, ld_scales, ts, given, st)
                 : launch_nv_lora<0, 0>(grid, lds_bytes, w, rows, k, ldw, lb, ldb, la, lda, rank, scale, codes,
                                        ld_codes, scales, ld_scales, ts, given, st);
}

}  // namespace fp4r
