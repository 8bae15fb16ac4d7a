// LoRA merge and MXFP4 re-quantization of a weight in one pass, for gfx950.
//
// After each policy update the adapted weights are re-quantized at run time
// for the next FP4 rollout (Sol-RL project page, "Two-Stage Pipeline",
// Stage 2; aitrends summary, Stage-2 paragraph: LoRA of rank 32, real-time
// re-quantization with no compile step). With W [N, K] (nn.Linear layout),
// B [N, r] and A [r, K] the kernel forms
//     acc = sum_j B[n, j] A[j, k]   (fp32 fma, j = 0 .. r-1 in order)
//     W'[n, k] = fma(s, acc, W[n, k])
// and quantizes W' by the MX rule, so the merged weight never goes to HBM.
//
// Work: one 256-thread workgroup per tile of 32 weight rows x 256 columns.
// The tile's slice of A ([r][256]) and rows of B ([32][r]) are staged in LDS
// as fp32; thread t owns column octet t % 32 of rows t / 32 + 8 i
// (i = 0..3), so a 32-block's 4 octets sit in 4 adjacent lanes of one row.
// Per adapter index j a lane reads 8 values of A (two 16-byte LDS reads, the
// same addresses in both lane halves) and 4 of B (broadcasts), then does 32
// fmas. The W octets are loaded before the staging, so their latency hides
// behind it. Compiled with -ffp-contract=off; every fma is explicit.
#include "quant_common.h"

namespace fp4r {
namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 32;
constexpr int kTileCols = 256;

template <int BF16>
__device__ __forceinline__ float load1(const void* p, int64_t i) {
  if (BF16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
  return reinterpret_cast<const float*>(p)[i];
}

// PANEL: the grid covers the padded extent (nrows = whole panels, ncols =
// whole 128-element chunks) and writes zero codes with scale byte 127 there,
// as the panel quantizer does.
template <int WBF16, int ABBF16, bool PANEL>
__global__ __launch_bounds__(kThreads) void quant_mx_lora_kernel(
    const void* __restrict__ w, int64_t rows, int64_t k, int64_t ldw, const void* __restrict__ lb, int64_t ldb,
    const void* __restrict__ la, int64_t lda, int rank, float scale, uint8_t* __restrict__ codes, int64_t ld_codes,
    uint8_t* __restrict__ scales, int64_t ld_scales, int64_t nrows, int64_t nc) {
  extern __shared__ float lds[];
  float* sa = lds;                        // [rank][kTileCols]
  float* sb = lds + rank * kTileCols;     // [kTileRows][rank]
  const int64_t r0 = (int64_t)blockIdx.y * kTileRows;
  const int64_t c0 = (int64_t)blockIdx.x * kTileCols;
  const int o = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int64_t og = (c0 >> 3) + o;            // global octet index along K
  const bool col_ok = og * 8 < k;              // shared by a 32-block's 4 octets (k % 32 == 0)

  float wv[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = r0 + rg + 8 * i;
    if (row < rows && col_ok) {
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

  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  for (int j = 0; j < rank; ++j) {
    const float4 a0 = *reinterpret_cast<const float4*>(sa + j * kTileCols + 8 * o);
    const float4 a1 = *reinterpret_cast<const float4*>(sa + j * kTileCols + 8 * o + 4);
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float bv = sb[(rg + 8 * i) * rank + j];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(bv, av[e], acc[i][e]);
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = r0 + rg + 8 * i;  // the same for a 32-block's 4 lanes
    if (row >= nrows) continue;
    const bool valid = row < rows && col_ok;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = valid ? fmaf(scale, acc[i][e], wv[i][e]) : 0.f;
    uint32_t S;
    const uint32_t wd = mx_block(v, S);
    if (PANEL) {
      if (og < nc * 16) {
        const int64_t blk = (row >> 8) * nc + (og >> 4), rr = row & 255;
        *reinterpret_cast<uint32_t*>(codes + (blk * 256 + rr) * 64 + (og & 15) * 4) = valid ? wd : 0u;
        if ((og & 3) == 0) scales[(blk * 256 + rr) * 4 + ((og & 15) >> 2)] = (uint8_t)(valid ? S : 127u);
      }
    } else if (valid) {
      *reinterpret_cast<uint32_t*>(codes + row * ld_codes + og * 4) = wd;
      if ((og & 3) == 0) scales[row * ld_scales + (og >> 2)] = (uint8_t)S;
    }
  }
}

template <int WBF16, int ABBF16, bool PANEL>
hipError_t launch_lora(dim3 grid, size_t lds_bytes, const void* w, int64_t rows, int64_t k, int64_t ldw,
                       const void* lb, int64_t ldb, const void* la, int64_t lda, int rank, float scale,
                       uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, int64_t nrows, int64_t nc,
                       hipStream_t st) {
  auto kernel = quant_mx_lora_kernel<WBF16, ABBF16, PANEL>;
  if (lds_bytes > 65536) {  // ranks above 56: more than the default dynamic LDS limit
    const hipError_t e =
        hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (e != hipSuccess) return e;
  }
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

}  // namespace fp4r
