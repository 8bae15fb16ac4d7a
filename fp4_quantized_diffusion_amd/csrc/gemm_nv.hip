// NVFP4-style x NVFP4-style GEMM (E2M1 codes, E4M3 scale per 16 along K,
// fp32 tensor scale per operand) with fp32 accumulation, for gfx950:
// the kernel for scale rows that are not 4-byte aligned. Aligned scale rows
// (the library's own quantizer output) take the persistent f16-MFMA kernel
// in gemm_mx.hip, which dequantizes with gfx950's scaled conversions.
//
// gfx950's scaled MFMA only takes power-of-two (E8M0) block scales, and an
// E2M1 code times an E4M3 scale needs up to 6 significant bits, more than
// FP8/FP6 hold. bf16 (8 significant bits) holds it exactly, so each fragment
// is dequantized in registers to bf16 -- G[m] * dec(S), exact -- and fed to
// V_MFMA_F32_16X16X32_BF16; the two tensor scales multiply the fp32 sum once
// in the epilogue. This runs at the BF16 MFMA rate.
//
// Layout and tiling follow the MXFP4 kernel: weight rows feed the MFMA's
// first operand (D row = n), activation rows its second (D column = m);
// 256 x 256 tiles, 4 waves of 128 x 128, 256-element K stages in LDS. For
// V_MFMA_F32_16X16X32_BF16, lane l holds row l % 16 and the 8 K-elements
// 8 (l / 16) .. 8 (l / 16) + 7 of a 32-element K step: 4 code bytes and one
// scale byte.
#include "gemm_common.h"

namespace fp4r {
namespace {

using namespace gemm;
constexpr int SB = 16;  // scale bytes per row per stage (256 / 16)

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float e4m3_value(uint32_t S) {
  const uint32_t e = S >> 3, m = S & 7u;
  return e == 0 ? (float)m * 0x1p-9f : ldexpf((float)(8u + m), (int)e - 10);
}

// bf16 bits of one E2M1 nibble's value (sign included).
__device__ __forceinline__ uint32_t e2m1_bf16(uint32_t nib) {
  const uint32_t m = nib & 7u;
  const uint32_t mag = m == 0 ? 0u : (m == 1 ? 0x3F00u : 0x3F80u + ((m - 2u) << 6));
  return mag | ((nib & 8u) << 12);
}

// 8 nibbles (one 32-bit word, element 2j in the low nibble of byte j) times
// the block scale -> 8 bf16 (exact), packed two per 32-bit word.
__device__ __forceinline__ v8bf dequant8(uint32_t w, float scale) {
  v4u out;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float lo = __uint_as_float(e2m1_bf16((w >> (8 * p)) & 15u) << 16) * scale;
    const float hi = __uint_as_float(e2m1_bf16((w >> (8 * p + 4)) & 15u) << 16) * scale;
    out[p] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
  }
  return __builtin_bit_cast(v8bf, out);
}

template <int BF16OUT, int RESID>
__global__ __launch_bounds__(kThreads, 1) void gemm_nv_bytes_kernel(
    const uint8_t* __restrict__ a, int64_t lda, const uint8_t* __restrict__ as, int64_t ld_as,
    const float* __restrict__ a_ts, const uint8_t* __restrict__ b, int64_t ldb, const uint8_t* __restrict__ bs,
    int64_t ld_bs, const float* __restrict__ b_ts, int M, int N, int K, void* __restrict__ c, int64_t ldc,
    const float* residual, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  Smem<SB>& s = *reinterpret_cast<Smem<SB>*>(smem_raw);

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, g = lane >> 4;

  const int kbytes = K >> 1;
  const int nstages = (kbytes + BKB - 1) / BKB;

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  Operand oa, ob;
  make_operand(oa, a, lda, as, ld_as, m0, M);
  make_operand(ob, b, ldb, bs, ld_bs, n0, N);

  Prefetch<SB> p;
  load_stage<SB>(p, oa, ob, 0, kbytes, 8);
  store_stage<SB>(s, 0, p);
  __syncthreads();

  for (int st = 0; st < nstages; ++st) {
    const int buf = st & 1;
    if (st + 1 < nstages) load_stage<SB>(p, oa, ob, (st + 1) * BKB, kbytes, 8);
#pragma unroll 2
    for (int kk = 0; kk < 8; ++kk) {
      const int coff = 16 * kk + 4 * g;        // code byte of this lane's 8 elements
      const int soff = 2 * kk + (g >> 1);      // their scale block within the stage
      v8bf fx[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int rm = wm * 128 + j * 16 + r16;
        const uint32_t w = *reinterpret_cast<const uint32_t*>(&s.a[buf][rm * ROWB + coff]);
        fx[j] = dequant8(w, e4m3_value(s.as[buf][rm * SB + soff]));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rn = wn * 128 + i * 16 + r16;
        const uint32_t w = *reinterpret_cast<const uint32_t*>(&s.b[buf][rn * ROWB + coff]);
        const v8bf fw = dequant8(w, e4m3_value(s.bs[buf][rn * SB + soff]));
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw, fx[j], acc[i][j], 0, 0, 0);
      }
    }
    if (st + 1 < nstages) store_stage<SB>(s, buf ^ 1, p);
    __syncthreads();
  }

  const float mul = (*a_ts) * (*b_ts);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      store_acc<BF16OUT, RESID>(acc[i][j], m0 + wm * 128 + j * 16 + r16, n0 + wn * 128 + i * 16 + 4 * g, M, N, c,
                                ldc, residual, mul);
}

template <int BF16OUT, int RESID>
hipError_t launch(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as, const float* a_ts,
                  const uint8_t* b, int64_t ldb, const uint8_t* bs, int64_t ld_bs, const float* b_ts, int64_t m,
                  int64_t n, int64_t k, void* c, int64_t ldc, const float* residual, hipStream_t st) {
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  const size_t smem = sizeof(Smem<SB>);
  auto kern = gemm_nv_bytes_kernel<BF16OUT, RESID>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  kern<<<(unsigned)(tiles_m * tiles_n), kThreads, smem, st>>>(a, lda, as, ld_as, a_ts, b, ldb, bs, ld_bs, b_ts,
                                                               (int)m, (int)n, (int)k, c, ldc, residual, tiles_m,
                                                               tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_nv(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as, const float* a_ts,
                          const uint8_t* b, int64_t ldb, const uint8_t* bs, int64_t ld_bs, const float* b_ts,
                          int64_t m, int64_t n, int64_t k, void* c, int c_bf16, int64_t ldc, const float* residual,
                          hipStream_t st) {
  if (ld_as % 4 == 0 && ld_bs % 4 == 0 && reinterpret_cast<uintptr_t>(as) % 4 == 0 &&
      reinterpret_cast<uintptr_t>(bs) % 4 == 0)
    return launch_gemm_nv_f16(a, lda, as, ld_as, a_ts, b, ldb, bs, ld_bs, b_ts, m, n, k, c, c_bf16, ldc, residual, st);
  if (c_bf16) return launch<1, 0>(a, lda, as, ld_as, a_ts, b, ldb, bs, ld_bs, b_ts, m, n, k, c, ldc, nullptr, st);
  if (residual) return launch<0, 1>(a, lda, as, ld_as, a_ts, b, ldb, bs, ld_bs, b_ts, m, n, k, c, ldc, residual, st);
  return launch<0, 0>(a, lda, as, ld_as, a_ts, b, ldb, bs, ld_bs, b_ts, m, n, k, c, ldc, nullptr, st);
}

}  // namespace fp4r
