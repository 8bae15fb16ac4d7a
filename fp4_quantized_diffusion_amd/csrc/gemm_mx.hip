// MXFP4 x MXFP4 GEMM with fp32 accumulation on gfx950's scaled MFMA.
//
// The solver linears of the FP4 rollout are FP4 x FP4 products at up to four
// times the BF16 rate (Sol-RL project page, "Two-Stage Pipeline"). Here
//     C[m, n] = sum_k A_hat[m, k] * B_hat[n, k]   (+ residual[m, n])
// with A the activation [M, K] and B the weight [N, K], both MXFP4 (E2M1
// codes, one E8M0 scale per 32 along K).
//
// Hardware mapping (gfx950, V_MFMA_SCALE_F32_16X16X128_F8F6F4 with FP4
// operands): lane l of a wave supplies row (l % 16) of its operand and the 32
// consecutive K-elements of K-block (l / 16) -- 16 packed bytes, exactly a
// slice of the row-major code layout -- plus that block's E8M0 scale byte.
// The accumulator holds D[4 (l / 16) + j][l % 16], j = 0..3.
//
// The WEIGHT rows feed the MFMA's first operand and the ACTIVATION rows its
// second, so D's row index is n and its column index is m: each lane then
// holds 4 consecutive n of one m row and stores them as one 16-byte (fp32)
// or 8-byte (bf16) vector.
//
// K order: a stage covers 8 K-blocks (256 elements, 128 bytes per row). For
// MFMA sub-step kk (0, 1) lane group g = l / 16 takes K-block 2g + kk, so a
// lane's two scales are adjacent bytes (one 16-bit LDS read; the MFMA's
// op_sel picks byte kk) and its codes are 32 contiguous bytes. Any
// permutation of K applied to both operands leaves the sum unchanged.
//
// Tiling: 256 x 256 output tile per 256-thread workgroup (4 waves, 2 x 2,
// 128 x 128 each: 8 x 8 MFMA tiles, 256 fp32 accumulators per lane).
// Stages are double-buffered in LDS; the next stage's global loads are in
// flight while the current stage's 128 MFMAs per wave run.
#include "gemm_common.h"

namespace fp4r {
namespace {

using namespace gemm;
constexpr int SB = 8;  // scale bytes per row per stage

template <int BF16OUT, int RESID>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_kernel(
    const uint8_t* __restrict__ a, int64_t lda, const uint8_t* __restrict__ as, int64_t ld_as,
    const uint8_t* __restrict__ b, int64_t ldb, const uint8_t* __restrict__ bs, int64_t ld_bs, int M, int N,
    int K, void* __restrict__ c, int64_t ldc, const float* residual, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  Smem<SB>& s = *reinterpret_cast<Smem<SB>*>(smem_raw);

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;  // the wave's 128 x 128 sub-tile
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
  load_stage<SB>(p, oa, ob, 0, kbytes, 16);
  store_stage<SB>(s, 0, p);
  __syncthreads();

  for (int st = 0; st < nstages; ++st) {
    const int buf = st & 1;
    if (st + 1 < nstages) load_stage<SB>(p, oa, ob, (st + 1) * BKB, kbytes, 16);

    // scales: 16-bit reads, byte kk selected by the MFMA's op_sel
    int sw[8], sx[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int rn = wn * 128 + f * 16 + r16;  // weight row (MFMA operand A)
      const int rm = wm * 128 + f * 16 + r16;  // activation row (MFMA operand B)
      sw[f] = *reinterpret_cast<const uint16_t*>(&s.bs[buf][rn * SB + 2 * g]);
      sx[f] = *reinterpret_cast<const uint16_t*>(&s.as[buf][rm * SB + 2 * g]);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int off = (2 * g + kk) * 16;
      v8i fx[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int rm = wm * 128 + j * 16 + r16;
        const uint4 qx = *reinterpret_cast<const uint4*>(&s.a[buf][rm * ROWB + off]);
        fx[j] = v8i{(int)qx.x, (int)qx.y, (int)qx.z, (int)qx.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rn = wn * 128 + i * 16 + r16;
        const uint4 qw = *reinterpret_cast<const uint4*>(&s.b[buf][rn * ROWB + off]);
        const v8i fw = v8i{(int)qw.x, (int)qw.y, (int)qw.z, (int)qw.w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (kk == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fw, fx[j], acc[i][j], 4, 4, 0, sw[i], 0,
                                                                         sx[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fw, fx[j], acc[i][j], 4, 4, 1, sw[i], 1,
                                                                         sx[j]);
        }
      }
    }
    if (st + 1 < nstages) store_stage<SB>(s, buf ^ 1, p);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      store_acc<BF16OUT, RESID>(acc[i][j], m0 + wm * 128 + j * 16 + r16, n0 + wn * 128 + i * 16 + 4 * g, M, N, c,
                                ldc, residual, 1.0f);
}

template <int BF16OUT, int RESID>
hipError_t launch(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as, const uint8_t* b, int64_t ldb,
                  const uint8_t* bs, int64_t ld_bs, int64_t m, int64_t n, int64_t k, void* c, int64_t ldc,
                  const float* residual, hipStream_t st) {
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  const size_t smem = sizeof(Smem<SB>);
  auto kern = gemm_mx_kernel<BF16OUT, RESID>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  kern<<<(unsigned)(tiles_m * tiles_n), kThreads, smem, st>>>(a, lda, as, ld_as, b, ldb, bs, ld_bs, (int)m, (int)n,
                                                               (int)k, c, ldc, residual, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as, const uint8_t* b,
                          int64_t ldb, const uint8_t* bs, int64_t ld_bs, int64_t m, int64_t n, int64_t k, void* c,
                          int c_bf16, int64_t ldc, const float* residual, hipStream_t st) {
  if (c_bf16) return launch<1, 0>(a, lda, as, ld_as, b, ldb, bs, ld_bs, m, n, k, c, ldc, nullptr, st);
  if (residual) return launch<0, 1>(a, lda, as, ld_as, b, ldb, bs, ld_bs, m, n, k, c, ldc, residual, st);
  return launch<0, 0>(a, lda, as, ld_as, b, ldb, bs, ld_bs, m, n, k, c, ldc, nullptr, st);
}

}  // namespace fp4r
