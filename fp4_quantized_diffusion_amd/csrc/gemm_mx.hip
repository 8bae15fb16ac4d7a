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
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef float v16f __attribute__((ext_vector_type(16)));

// K stage = 128 elements: 64 code bytes and 4 scale bytes per row.
constexpr int KSTAGE_B = 64;
constexpr int SCB = 4;
constexpr int NBUF = 4;      // LDS stage buffers: three stages in flight while one is consumed

// One K stage in LDS: codes of both operands and their scale bytes, all
// written by direct global->LDS loads. The stage buffers are separate
// objects, so the compiler can see that reading one never depends on the
// loads in flight into another.
struct __attribute__((aligned(16))) StageMx {
  uint8_t a[BM * KSTAGE_B];
  uint8_t b[BN * KSTAGE_B];
  uint8_t as[BM * SCB];
  uint8_t bs[BN * SCB];
};
constexpr int kEpiRow = 272;  // epilogue staging row stride (bytes): 256 B of bf16 + 16 B against conflicts

// 16-byte chunk c (0..3) of row r lives at position c ^ ((r >> 2) & 3): the
// 16 rows of a fragment read then cover every (r % 4, position) pair, i.e.
// all 64 LDS banks, without conflicts.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 2) & 3); }

struct OperandMx {
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t off[4];   // this lane's chunk for each of the wave's 4 code loads of a stage
  uint32_t soff;     // this lane's scale word / byte of a stage
};

// Code loads: wave w's load `it` fills LDS rows 16 (4 w + it) .. +15 (1 KB);
// lane L writes position L % 4 of row 16 (4 w + it) + L / 4, i.e. global
// chunk (L % 4) ^ swizzle. Scales: thread t handles row t. With 4-byte
// aligned scale rows (SDW) the stage's 4 scale bytes are one word, loaded
// straight into LDS (a wave fills rows 64 w .. +63); otherwise the thread
// loads the 4 bytes into registers and writes the word to LDS itself.
template <bool SDW>
__device__ __forceinline__ void make_operand_mx(OperandMx& o, const uint8_t* codes, int64_t ld, const uint8_t* scales,
                                                int64_t ld_s, int row0, int rows) {
  const int valid = min(rows - row0, 256);
  o.codes = make_rsrc(codes + (int64_t)row0 * ld, (int64_t)valid * ld);
  o.scales = make_rsrc(scales + (int64_t)row0 * ld_s, (int64_t)valid * ld_s);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = (w * 4 + it) * 16 + (lane >> 2);
    o.off[it] = (uint32_t)(r * ld + swz(r, lane & 3) * 16);
  }
  o.soff = (uint32_t)((w * 64 + lane) * ld_s);  // this thread's scale row (both paths)
}

// Issue stage `st` into `dst`. Code chunks at or past the row's code length
// read as zero (out-of-range offset): zero codes contribute nothing whatever
// their scale. Without SDW the scale bytes come back in sc[] (issued first,
// so they complete before this stage's code loads) and are written to LDS
// by store_scale_regs().
template <bool SDW>
__device__ __forceinline__ void issue_stage(StageMx& dst, const OperandMx& oa, const OperandMx& ob, int st,
                                            int kbytes, uint32_t sc[8]) {
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = st * KSTAGE_B;
  const int kblk = st * SCB, nblk = kbytes >> 4;
  if (!SDW) {
#pragma unroll
    for (int j = 0; j < SCB; ++j) {
      const bool in = kblk + j < nblk;
      sc[j] = __builtin_amdgcn_raw_buffer_load_b8(oa.scales, in ? oa.soff + j : kOob, kblk, 0);
      sc[SCB + j] = __builtin_amdgcn_raw_buffer_load_b8(ob.scales, in ? ob.soff + j : kOob, kblk, 0);
    }
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = (w * 4 + it) * 16 + (lane >> 2);
    const bool kin = kb + swz(r, lane & 3) * 16 < kbytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(oa.codes, (lds_ptr_t)(dst.a + (w * 4 + it) * 1024), 16,
                                             kin ? oa.off[it] : kOob, kb, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ob.codes, (lds_ptr_t)(dst.b + (w * 4 + it) * 1024), 16,
                                             kin ? ob.off[it] : kOob, kb, 0, 0);
  }
  if (SDW) {
    // whole words: bytes past the block count (inside the row's padding) are
    // neutralised when the fragments are read
    const bool in = kblk < nblk;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(oa.scales, (lds_ptr_t)(dst.as + w * 256), 4, in ? oa.soff : kOob,
                                             kblk, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ob.scales, (lds_ptr_t)(dst.bs + w * 256), 4, in ? ob.soff : kOob,
                                             kblk, 0, 0);
  }
}

__device__ __forceinline__ void store_scale_regs(StageMx& dst, const uint32_t sc[8]) {
  *reinterpret_cast<uint32_t*>(&dst.as[threadIdx.x * SCB]) = sc[0] | (sc[1] << 8) | (sc[2] << 16) | (sc[3] << 24);
  *reinterpret_cast<uint32_t*>(&dst.bs[threadIdx.x * SCB]) = sc[4] | (sc[5] << 8) | (sc[6] << 16) | (sc[7] << 24);
}

// The lane's two scale bytes (K-blocks 2h, 2h+1 of stage st) with blocks
// past the end replaced by 127 (2^0): their codes are zero, but a stray
// 0xFF (NaN) scale byte from row padding must not reach the MFMA.
__device__ __forceinline__ int clean_scales(int v, int st, int nblk, int h) {
  const int b0 = st * SCB + 2 * h;
  if (b0 + 1 < nblk) return v;
  if (b0 < nblk) return (v & 0xFF) | 0x7F00;
  return 0x7F7F;
}

template <int KS>
__device__ __forceinline__ v16f mfma_ks(v8i w, v8i x, v16f acc, int sw, int sx) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, x, acc, 4, 4, KS, sw, KS, sx);
}

// Fragments of K step ks: lane half h takes K-block 2h + ks of the stage.
template <int KS>
__device__ __forceinline__ void read_frags(const StageMx& cur, int rn0, int rm0, int h, v8i fw[4], v8i fx[4]) {
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int rn = rn0 + f * 32, rm = rm0 + f * 32;
    const uint4 qw = *reinterpret_cast<const uint4*>(&cur.b[rn * KSTAGE_B + swz(rn, 2 * h + KS) * 16]);
    const uint4 qx = *reinterpret_cast<const uint4*>(&cur.a[rm * KSTAGE_B + swz(rm, 2 * h + KS) * 16]);
    fw[f] = v8i{(int)qw.x, (int)qw.y, (int)qw.z, (int)qw.w, 0, 0, 0, 0};
    fx[f] = v8i{(int)qx.x, (int)qx.y, (int)qx.z, (int)qx.w, 0, 0, 0, 0};
  }
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding (and all of its LDS operations are done).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}

// Consume stage `st` from `cur` while stage st + 3 streams into `refill`.
template <bool SDW>
__device__ __forceinline__ void stage_step(v16f acc[4][4], StageMx& cur, StageMx& refill, int st, const OperandMx& oa,
                                           const OperandMx& ob, int kbytes, int rn0, int rm0, int h) {
  constexpr int PER = SDW ? 10 : 16;     // vector-memory instructions per wave per stage
  wait_vm_lgkm0<2 * PER>();              // this wave's share of stage st has landed
  // ... everyone's has, and nobody still reads `refill`. A bare barrier: the
  // release fence of __syncthreads() would also wait for the two younger
  // stages still in flight.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  uint32_t sc[8];
  issue_stage<SDW>(refill, oa, ob, st + 3, kbytes, sc);
  const int nblk = kbytes >> 4;
  int sw[4], sx[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    sw[f] = clean_scales(*reinterpret_cast<const uint16_t*>(&cur.bs[(rn0 + f * 32) * SCB + 2 * h]), st, nblk, h);
    sx[f] = clean_scales(*reinterpret_cast<const uint16_t*>(&cur.as[(rm0 + f * 32) * SCB + 2 * h]), st, nblk, h);
  }
  v8i f0w[4], f0x[4], f1w[4], f1x[4];
  read_frags<0>(cur, rn0, rm0, h, f0w, f0x);
  read_frags<1>(cur, rn0, rm0, h, f1w, f1x);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mfma_ks<0>(f0w[i], f0x[j], acc[i][j], sw[i], sx[j]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mfma_ks<1>(f1w[i], f1x[j], acc[i][j], sw[i], sx[j]);
  if (!SDW) {
    // the scale bytes were issued before this stage's code loads: once only
    // those 8 remain, the bytes are in registers
    asm volatile("" ::: "memory");
    wait_vm_lgkm0<8>();
    store_scale_regs(refill, sc);
  }
}

// Main kernel. MFMA: V_MFMA_SCALE_F32_32X32X64_F8F6F4 with FP4 operands --
// lane l supplies row l % 32 and the 32 K-elements of K-block l / 32 of a
// 64-element K step, plus that block's scale byte; the accumulator holds
// D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32], r = 0..15. Weight rows feed the
// MFMA's first operand, so D's row index is n and its column index m.
// K order within a 128-element stage: K step ks (0, 1) gives lane half h
// K-block 2h + ks, so a lane's code bytes are 32 contiguous bytes and its two
// scale bytes one 16-bit word (the MFMA's op_sel picks byte ks).
template <int BF16OUT, int RESID, bool SDW>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_kernel(
    const uint8_t* __restrict__ a, int64_t lda, const uint8_t* __restrict__ as, int64_t ld_as,
    const uint8_t* __restrict__ b, int64_t ldb, const uint8_t* __restrict__ bs, int64_t ld_bs, int M, int N,
    int K, void* __restrict__ c, int64_t ldc, const float* residual, int tiles_m, int tiles_n) {
  __shared__ StageMx s0, s1, s2, s3;

  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // the wave's 128 x 128 sub-tile
  const int r32 = lane & 31, h = lane >> 5;
  const int rn0 = wn * 128 + r32, rm0 = wm * 128 + r32;

  const int kbytes = K >> 1;
  const int nstages = (kbytes + KSTAGE_B - 1) / KSTAGE_B;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  OperandMx oa, ob;
  make_operand_mx<SDW>(oa, a, lda, as, ld_as, m0, M);
  make_operand_mx<SDW>(ob, b, ldb, bs, ld_bs, n0, N);

  // prologue: stages 0..2 in flight (stages past the end read zeros). The
  // stage waits count this wave's loads in issue order, so no load may be
  // moved across a stage boundary.
  {
    uint32_t sc[8];
    issue_stage<SDW>(s0, oa, ob, 0, kbytes, sc);
    asm volatile("" ::: "memory");
    if (!SDW) { wait_vm_lgkm0<8>(); store_scale_regs(s0, sc); }
    issue_stage<SDW>(s1, oa, ob, 1, kbytes, sc);
    asm volatile("" ::: "memory");
    if (!SDW) { wait_vm_lgkm0<8>(); store_scale_regs(s1, sc); }
    issue_stage<SDW>(s2, oa, ob, 2, kbytes, sc);
    asm volatile("" ::: "memory");
    if (!SDW) { wait_vm_lgkm0<8>(); store_scale_regs(s2, sc); }
  }
  // The stage count is rounded up to a multiple of 4 (the ring size); the
  // extra stages hold only zero codes and add nothing. One exit keeps the
  // accumulators in place.
  for (int st = 0; st < nstages; st += NBUF) {
    stage_step<SDW>(acc, s0, s3, st, oa, ob, kbytes, rn0, rm0, h);
    stage_step<SDW>(acc, s1, s0, st + 1, oa, ob, kbytes, rn0, rm0, h);
    stage_step<SDW>(acc, s2, s1, st + 2, oa, ob, kbytes, rn0, rm0, h);
    stage_step<SDW>(acc, s3, s2, st + 3, oa, ob, kbytes, rn0, rm0, h);
  }
  __builtin_amdgcn_s_waitcnt(0);  // drain the trailing (past-the-end) loads before LDS is reused
  __syncthreads();

  // Epilogue: stage the wave's 128 x 128 tile through LDS so global stores
  // are 16-byte vectors covering whole 256/512-byte row segments.
  int me = m0 + wm * 128, ne = n0 + wn * 128;
  float one = 1.0f;  // opaque to the compiler: keeps epilogue work out of the main loop
  asm volatile("" : "+v"(me), "+v"(ne), "+v"(one));
  uint8_t* stage = (wave == 0 ? s0.a : wave == 1 ? s1.a : wave == 2 ? s2.a : s3.a);
  constexpr int ESZ = BF16OUT ? 2 : 4;
  constexpr int ROWS_PER_PASS = BF16OUT ? 64 : 32;
  constexpr int ROWBYTES = 128 * ESZ;
  constexpr int PITCH = ROWBYTES + 16;
  static_assert(ROWS_PER_PASS * PITCH <= (int)sizeof(StageMx), "epilogue pass must fit in one stage buffer");
#pragma unroll
  for (int pass = 0; pass < 128 / ROWS_PER_PASS; ++pass) {
    // accumulators -> LDS: m-row = 32 j + r32 (within the pass), n = 32 i + 8 q + 4 h + 0..3
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 32 * j + r32 - pass * ROWS_PER_PASS;
      if (32 * j < pass * ROWS_PER_PASS || 32 * j >= (pass + 1) * ROWS_PER_PASS) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = 32 * i + 8 * q + 4 * h;
          const float v0 = acc[i][j][4 * q] * one, v1 = acc[i][j][4 * q + 1] * one;
          const float v2 = acc[i][j][4 * q + 2] * one, v3 = acc[i][j][4 * q + 3] * one;
          uint8_t* dst = stage + row * PITCH + n * ESZ;
          if (BF16OUT) {
            *reinterpret_cast<uint2*>(dst) =
                make_uint2((uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16),
                           (uint32_t)f32_to_bf16(v2) | ((uint32_t)f32_to_bf16(v3) << 16));
          } else {
            *reinterpret_cast<float4*>(dst) = make_float4(v0, v1, v2, v3);
          }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // LDS -> global: each lane moves 16 bytes; a wave instruction covers whole rows
    constexpr int CH_PER_ROW = ROWBYTES / 16;
    constexpr int ITERS = ROWS_PER_PASS * CH_PER_ROW / 64;
#pragma unroll 4
    for (int t = 0; t < ITERS; ++t) {
      const int id = t * 64 + lane;
      const int row = id / CH_PER_ROW, ch = id % CH_PER_ROW;
      const int m = me + pass * ROWS_PER_PASS + row;
      const int n = ne + ch * (16 / ESZ);
      const uint4 v = *reinterpret_cast<const uint4*>(stage + row * PITCH + ch * 16);
      if (m >= M || n >= N) continue;
      const int64_t off = (int64_t)m * ldc + n;
      if (n + 16 / ESZ <= N) {
        if (BF16OUT) {
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(c) + off) = v;
        } else {
          float4 o = __builtin_bit_cast(float4, v);
          if (RESID) {
            const float4 r = *reinterpret_cast<const float4*>(residual + off);
            o.x += r.x; o.y += r.y; o.z += r.z; o.w += r.w;
          }
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(c) + off) = o;
        }
      } else {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
        for (int e = 0; e < 16 / ESZ && n + e < N; ++e) {
          if (BF16OUT) {
            reinterpret_cast<uint16_t*>(c)[off + e] = (uint16_t)(wv[e / 2] >> (16 * (e & 1)));
          } else {
            float o = __uint_as_float(wv[e]);
            if (RESID) o += residual[off + e];
            reinterpret_cast<float*>(c)[off + e] = o;
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
  }
}

template <int BF16OUT, int RESID>
hipError_t launch(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as, const uint8_t* b, int64_t ldb,
                  const uint8_t* bs, int64_t ld_bs, int64_t m, int64_t n, int64_t k, void* c, int64_t ldc,
                  const float* residual, hipStream_t st) {
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  const unsigned grid = (unsigned)(tiles_m * tiles_n);
  // scales as whole 4-byte words when every row's scale bytes start 4-byte aligned
  const bool sdw = (ld_as % 4 == 0) && (ld_bs % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(as) % 4 == 0) && (reinterpret_cast<uintptr_t>(bs) % 4 == 0);
  if (sdw)
    gemm_mx_kernel<BF16OUT, RESID, true><<<grid, kThreads, 0, st>>>(a, lda, as, ld_as, b, ldb, bs, ld_bs, (int)m,
                                                                    (int)n, (int)k, c, ldc, residual, tiles_m, tiles_n);
  else
    gemm_mx_kernel<BF16OUT, RESID, false><<<grid, kThreads, 0, st>>>(a, lda, as, ld_as, b, ldb, bs, ld_bs, (int)m,
                                                                     (int)n, (int)k, c, ldc, residual, tiles_m, tiles_n);
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
