// MXFP4 x MXFP4 GEMM with fp32 accumulation on gfx950's scaled MFMA.
//
// The solver linears of the FP4 rollout are FP4 x FP4 products at up to four
// times the BF16 rate (Sol-RL project page, "Two-Stage Pipeline"). Here
//     C[m, n] = sum_k A_hat[m, k] * B_hat[n, k]   (+ residual[m, n])
// with A the activation [M, K] and B the weight [N, K], both MXFP4 (E2M1
// codes, one E8M0 scale per 32 along K).
//
// Design (gfx950):
//  * MFMA: V_MFMA_SCALE_F32_32X32X64_F8F6F4 with FP4 operands. Lane l
//    supplies row l % 32 and the 32 K-elements of K-block l / 32 of a
//    64-element K step (16 packed bytes -- a slice of the row-major code
//    layout) plus that block's E8M0 byte; the accumulator holds
//    D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32], r = 0..15. Weight rows feed
//    the MFMA's first operand, so D's row index is n and its column index m.
//  * K order: a 128-element K stage is two K steps; in step ks lane half
//    h = l / 32 takes K-block 2h + ks, so a lane's codes for the stage are 32
//    contiguous bytes and its two scale bytes one 16-bit word (the MFMA's
//    op_sel picks byte ks). Any K permutation applied to both operands leaves
//    the sum unchanged.
//  * Tiles: 256 x 256 outputs per 256-thread workgroup (4 waves of 128 x 128:
//    4 x 4 MFMA tiles, 256 fp32 accumulators per lane in AGPRs).
//  * Persistent: one workgroup per CU walks a sequence of tiles; its K
//    stages form one stream across tiles. A ring of four LDS stage buffers
//    keeps three stages in flight, filled by direct global->LDS buffer loads
//    (no registers), so the next tile's first stages arrive while the
//    current tile finishes and its epilogue runs.
//  * Each pipeline step waits for the next stage, issues the stage four
//    ahead, and runs the current stage's MFMAs from registers while the next
//    stage's fragments are read from LDS.
//  * Epilogue straight from registers: one lane-half swap (v_permlane32_swap)
//    gives every lane 16 consecutive n of its m row, stored as 16-byte vectors.
//  * Operand layouts: row-major (any leading dimension) or the panel layout,
//    where each 256-row x 128-element (panel, K chunk) pair is one contiguous
//    16 KiB block of codes and a 1 KiB block of scales. Every stage load of
//    the panel layout is a contiguous 1 KiB run per instruction; row-major
//    rows give 64-byte pieces of 16 rows (codes) and single bytes or words of
//    64 rows (scales), which costs the CU's load path about 2.5x the cycles
//    per stage.
//  * Tile order: workgroups are dispatched round-robin over the 8 XCDs; the
//    tile map gives each XCD a contiguous band of tiles, walked in groups of
//    kGroupM tile-rows, so tiles that run together on an XCD share A and B
//    panels in its L2.
#include <mutex>

#include "gemm_common.h"
#include "mx_common.h"

namespace fp4r {
namespace {

using namespace gemm;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int KSTAGE_B = 64;  // code bytes per row per K stage (128 elements)
constexpr int SCB = 4;        // MX scale bytes per row per K stage
constexpr int SCB_NV = 8;     // NVFP4-style scale bytes per row per K stage
constexpr int NBUF = 4;       // LDS stage buffers

// One K stage in LDS. The buffers are separate objects, so the compiler can
// see that reading one never depends on the loads in flight into another.
template <int SCBY>
struct __attribute__((aligned(16))) StageT {
  uint8_t a[BM * KSTAGE_B];
  uint8_t b[BN * KSTAGE_B];
  uint8_t as[BM * SCBY];
  uint8_t bs[BN * SCBY];
};
typedef StageT<SCB> StageMx;

// 16-byte chunk c (0..3) of row r lives at position c ^ ((r >> 2) & 3): the
// 16 rows of a fragment read then cover every (r % 4, position) pair, i.e.
// all 64 LDS banks, without conflicts.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 2) & 3); }

// Operand layout (kernel template parameter).
enum Layout {
  LD_ROW_BYTE = 0,  // row-major, scale rows of any alignment (bytes through registers)
  LD_ROW_WORD = 1,  // row-major, scale rows 4-byte aligned (direct word loads)
  LD_PANEL = 2,     // panel layout
  LD_NV = 3,        // NVFP4-style, row-major, scale rows 4-byte aligned (direct word loads)
};

template <int LD>
using Stage = StageT<LD == LD_NV ? SCB_NV : SCB>;

// Problem description shared by every step.
struct Problem {
  const uint8_t *a, *as, *b, *bs;
  const float *a_ts, *b_ts;        // NVFP4-style tensor scales
  int a_rpg;                       //   A's rows per tensor-scale group (0: one scale for all of A)
  const float* ex;                 // Euler epilogue: the state x, and the step dt
  float dt;
  const float* ru;                 // Euler + reward epilogue: the reward weights u [N]
  float* rp;                       //   and the per-wave partial sums [tiles][4]
  uint8_t *qc, *qs;                // GELU + MXFP4 epilogue: output codes / scales (panel layout)
  int qnc;                         //   and the output's 128-element chunks per panel row (n / 128)
  int64_t lda, ld_as, ldb, ld_bs;  // row-major layouts
  int M, N, kbytes, nblk;
  int nkc;                         // K chunks of 128 elements (stages per tile)
  int tiles_m, tiles_n, total;
};

constexpr int kPanelCodeBlock = BM * KSTAGE_B;  // 16 KiB: one (panel, chunk) code block
constexpr int kPanelScaleBlock = BM * SCB;      // 1 KiB: its scale block

// This thread's share of a stage load, independent of the tile: code chunk
// offsets for its 4 code loads per operand (wave w's load `it` fills LDS rows
// 16 (4 w + it) .. +15; lane L writes position L % 4 of row
// 16 (4 w + it) + L / 4) and its scale row (row t). NVFP4-style stages have
// 8 scale bytes per row, loaded as two 4-byte words per thread: word j of
// wave w's lane L is word L % 2 of row 128 j + 32 w + L / 2, so each load of
// a wave fills 256 contiguous LDS bytes in row order (sa2 / sb2: the second
// load's offsets).
struct LaneOffsets {
  uint32_t ca[4], cb[4];
  uint32_t sa, sb;
  uint32_t sa2, sb2;
};

template <int LD>
__device__ __forceinline__ void make_lane_offsets(LaneOffsets& o, const Problem& p) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t lda = LD == LD_PANEL ? KSTAGE_B : p.lda, ldb = LD == LD_PANEL ? KSTAGE_B : p.ldb;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = (w * 4 + it) * 16 + (lane >> 2);
    o.ca[it] = (uint32_t)(r * lda + swz(r, lane & 3) * 16);
    o.cb[it] = (uint32_t)(r * ldb + swz(r, lane & 3) * 16);
  }
  o.sa = (uint32_t)(threadIdx.x * (LD == LD_PANEL ? SCB : p.ld_as));
  o.sb = (uint32_t)(threadIdx.x * (LD == LD_PANEL ? SCB : p.ld_bs));
  o.sa2 = o.sb2 = 0;
  if (LD == LD_NV) {
    const int r = w * 32 + (lane >> 1), wo = (lane & 1) * 4;
    o.sa = (uint32_t)(r * p.ld_as + wo);
    o.sb = (uint32_t)(r * p.ld_bs + wo);
    o.sa2 = (uint32_t)((r + 128) * p.ld_as + wo);
    o.sb2 = (uint32_t)((r + 128) * p.ld_bs + wo);
  }
}

// Buffer resources of one tile's operands (uniform, in SGPRs). Loads past
// the matrix (rows past M / N, a tile past the last) read as zero through
// the buffer range check. A panel-layout resource spans the tile's whole
// panel (every K chunk); its padding rows hold zero codes.
struct TileDesc {
  __amdgpu_buffer_rsrc_t a, b, as, bs;
};

template <int LD>
__device__ __forceinline__ TileDesc make_desc(const Problem& p, int pid) {
  int tm = 0, tn = 0;
  const bool live = pid < p.total;
  if (live) tile_coords(pid, p.tiles_m, p.tiles_n, tm, tn);
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  TileDesc d;
  if (LD == LD_PANEL) {
    const int64_t cb = live ? (int64_t)p.nkc * kPanelCodeBlock : 0, sb = live ? (int64_t)p.nkc * kPanelScaleBlock : 0;
    d.a = make_rsrc(p.a + tm * (int64_t)p.nkc * kPanelCodeBlock, cb);
    d.b = make_rsrc(p.b + tn * (int64_t)p.nkc * kPanelCodeBlock, cb);
    d.as = make_rsrc(p.as + tm * (int64_t)p.nkc * kPanelScaleBlock, sb);
    d.bs = make_rsrc(p.bs + tn * (int64_t)p.nkc * kPanelScaleBlock, sb);
    return d;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t va = live ? min(p.M - m0, BM) : 0, vb = live ? min(p.N - n0, BN) : 0;
  d.a = make_rsrc(p.a + (int64_t)m0 * p.lda, va * p.lda);
  d.b = make_rsrc(p.b + (int64_t)n0 * p.ldb, vb * p.ldb);
  d.as = make_rsrc(p.as + (int64_t)m0 * p.ld_as, va * p.ld_as);
  d.bs = make_rsrc(p.bs + (int64_t)n0 * p.ld_bs, vb * p.ld_bs);
  return d;
}

// Issue K stage `st` of the tile described by `d` into `dst`. Code bytes
// past K read as zero (out-of-range offset): zero codes contribute nothing
// whatever their scale. With byte scales (row-major, rows not 4-byte
// aligned) the scale bytes come back in sc[] -- issued first, so they
// complete before this stage's code loads -- and are written to LDS by
// store_scale_regs(). Panel layout: stage st is block st of the panel, and
// stages past the last chunk read as zero codes with zero scale bytes.
template <int LD>
__device__ __forceinline__ void issue_stage(Stage<LD>& dst, const Problem& p, const LaneOffsets& o, const TileDesc& d,
                                            int st, uint32_t sc[8]) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (LD == LD_NV) {
    // codes as in the row-major MX layout; scale bytes st*8 .. st*8+7 of
    // each row as two words (bytes past the row's blocks are masked when
    // the fragments are read)
    const int lane = threadIdx.x & 63;
    const int kb = st * KSTAGE_B, kblk = st * SCB_NV;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = (w * 4 + it) * 16 + (lane >> 2);
      const bool kin = kb + swz(r, lane & 3) * 16 < p.kbytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(d.a, (lds_ptr_t)(dst.a + (w * 4 + it) * 1024), 16,
                                               kin ? o.ca[it] : kOob, kb, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(d.b, (lds_ptr_t)(dst.b + (w * 4 + it) * 1024), 16,
                                               kin ? o.cb[it] : kOob, kb, 0, 0);
    }
    const bool in = kblk + (lane & 1) * 4 < p.nblk;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.as, (lds_ptr_t)(dst.as + w * 256), 4, in ? o.sa : kOob, kblk, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.as, (lds_ptr_t)(dst.as + 1024 + w * 256), 4, in ? o.sa2 : kOob, kblk,
                                             0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.bs, (lds_ptr_t)(dst.bs + w * 256), 4, in ? o.sb : kOob, kblk, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.bs, (lds_ptr_t)(dst.bs + 1024 + w * 256), 4, in ? o.sb2 : kOob, kblk,
                                             0, 0);
    return;
  }
  if (LD == LD_PANEL) {
    const bool in = st < p.nkc;  // uniform
    const int cboff = st * kPanelCodeBlock, sboff = st * kPanelScaleBlock;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(d.a, (lds_ptr_t)(dst.a + (w * 4 + it) * 1024), 16,
                                               in ? o.ca[it] : kOob, cboff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(d.b, (lds_ptr_t)(dst.b + (w * 4 + it) * 1024), 16,
                                               in ? o.cb[it] : kOob, cboff, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.as, (lds_ptr_t)(dst.as + w * 256), 4, in ? o.sa : kOob, sboff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.bs, (lds_ptr_t)(dst.bs + w * 256), 4, in ? o.sb : kOob, sboff, 0, 0);
    return;
  }
  constexpr bool SDW = LD == LD_ROW_WORD;
  const int lane = threadIdx.x & 63;
  const int kb = st * KSTAGE_B, kblk = st * SCB;
  if (!SDW) {
#pragma unroll
    for (int j = 0; j < SCB; ++j) {
      const bool in = kblk + j < p.nblk;
      sc[j] = __builtin_amdgcn_raw_buffer_load_b8(d.as, in ? o.sa + j : kOob, kblk, 0);
      sc[SCB + j] = __builtin_amdgcn_raw_buffer_load_b8(d.bs, in ? o.sb + j : kOob, kblk, 0);
    }
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = (w * 4 + it) * 16 + (lane >> 2);
    const bool kin = kb + swz(r, lane & 3) * 16 < p.kbytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.a, (lds_ptr_t)(dst.a + (w * 4 + it) * 1024), 16,
                                             kin ? o.ca[it] : kOob, kb, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.b, (lds_ptr_t)(dst.b + (w * 4 + it) * 1024), 16,
                                             kin ? o.cb[it] : kOob, kb, 0, 0);
  }
  if (SDW) {
    // whole 4-byte words (a wave fills rows 64 w .. +63); bytes past the
    // block count lie in the row and are neutralised when fragments are read
    const bool in = kblk < p.nblk;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.as, (lds_ptr_t)(dst.as + w * 256), 4, in ? o.sa : kOob, kblk, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.bs, (lds_ptr_t)(dst.bs + w * 256), 4, in ? o.sb : kOob, kblk, 0, 0);
  }
}

template <class St>
__device__ __forceinline__ void store_scale_regs(St& dst, const uint32_t sc[8]) {
  *reinterpret_cast<uint32_t*>(&dst.as[threadIdx.x * SCB]) = sc[0] | (sc[1] << 8) | (sc[2] << 16) | (sc[3] << 24);
  *reinterpret_cast<uint32_t*>(&dst.bs[threadIdx.x * SCB]) = sc[4] | (sc[5] << 8) | (sc[6] << 16) | (sc[7] << 24);
}

// The lane's two scale bytes (K-blocks 2h, 2h+1 of stage st) with blocks
// past the end replaced by 127 (2^0): their codes are zero, but a stray
// 0xFF (NaN) byte from row padding must not reach the MFMA.
__device__ __forceinline__ int clean_scales(int v, int st, int nblk, int h) {
  const int b0 = st * SCB + 2 * h;
  if (b0 + 1 < nblk) return v;
  if (b0 < nblk) return (v & 0xFF) | 0x7F00;
  return 0x7F7F;
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding and all of its LDS operations are done.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}

// "Wait until at most N of this wave's vector-memory operations are
// outstanding and its LDS operations are done, then barrier" as ONE asm
// block, so the wait cannot be scheduled after the barrier: a wave must not
// signal the barrier before its own loads into the stage the others are
// about to read have landed. No release fence (unlike __syncthreads(), whose
// fence would also wait for the younger stages still in flight); the memory
// clobber keeps the compiler from moving memory operations across it.
#define FP4R_WAIT_BARRIER(N) asm volatile("s_waitcnt vmcnt(" #N ") lgkmcnt(0)\n\ts_barrier" ::: "memory")
template <int N>
__device__ __forceinline__ void wait_barrier() {
  if constexpr (N == 20) FP4R_WAIT_BARRIER(20);
  else if constexpr (N == 30) FP4R_WAIT_BARRIER(30);
  else if constexpr (N == 24) FP4R_WAIT_BARRIER(24);
  else if constexpr (N == 32) FP4R_WAIT_BARRIER(32);
  else if constexpr (N == 36) FP4R_WAIT_BARRIER(36);
  else if constexpr (N == 48) FP4R_WAIT_BARRIER(48);
  else if constexpr (N == 52) FP4R_WAIT_BARRIER(52);
  else if constexpr (N == 56) FP4R_WAIT_BARRIER(56);
  else if constexpr (N == 63) FP4R_WAIT_BARRIER(63);
  else static_assert(N < 0, "add this vmcnt value");
}
#undef FP4R_WAIT_BARRIER

// All of one stage's fragments for this lane: scales and both K steps' codes.
struct Frags {
  int sw[4], sx[4];
  v8i w0[4], x0[4], w1[4], x1[4];
};

template <int KS, class St>
__device__ __forceinline__ void read_codes(const St& cur, int rn0, int rm0, int h, v8i fw[4], v8i fx[4]) {
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int rn = rn0 + f * 32, rm = rm0 + f * 32;
    const uint4 qw = *reinterpret_cast<const uint4*>(&cur.b[rn * KSTAGE_B + swz(rn, 2 * h + KS) * 16]);
    const uint4 qx = *reinterpret_cast<const uint4*>(&cur.a[rm * KSTAGE_B + swz(rm, 2 * h + KS) * 16]);
    fw[f] = v8i{(int)qw.x, (int)qw.y, (int)qw.z, (int)qw.w, 0, 0, 0, 0};
    fx[f] = v8i{(int)qx.x, (int)qx.y, (int)qx.z, (int)qx.w, 0, 0, 0, 0};
  }
}

// NVFP4-style: the lane's four scale bytes (blocks 4h .. 4h+3 of stage st,
// i.e. those of its chunks 2h and 2h+1) with blocks past the end set to 0.
// The GEMM multiplies every code by its block's scale, so a zero scale
// makes the (zero) codes past K and whatever lies in the row padding
// contribute exactly nothing.
__device__ __forceinline__ int clean_scales_nv(int v, int st, int nblk, int h) {
  const int b0 = st * SCB_NV + 4 * h;
  if (b0 + 4 <= nblk) return v;
  if (b0 >= nblk) return 0;
  return (int)((uint32_t)v & ((1u << (8 * (nblk - b0))) - 1u));
}

// Panel layout: the padding scale bytes are 127 and stages past the last
// chunk read as zero, so no byte needs replacing.
template <int LD>
__device__ __forceinline__ void read_stage(const Stage<LD>& cur, int st, int nblk, int rn0, int rm0, int h, Frags& f) {
  if (LD == LD_NV) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f.sw[q] = clean_scales_nv(*reinterpret_cast<const int*>(&cur.bs[(rn0 + q * 32) * SCB_NV + 4 * h]), st, nblk, h);
      f.sx[q] = clean_scales_nv(*reinterpret_cast<const int*>(&cur.as[(rm0 + q * 32) * SCB_NV + 4 * h]), st, nblk, h);
    }
    read_codes<0>(cur, rn0, rm0, h, f.w0, f.x0);
    read_codes<1>(cur, rn0, rm0, h, f.w1, f.x1);
    return;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int vw = *reinterpret_cast<const uint16_t*>(&cur.bs[(rn0 + q * 32) * SCB + 2 * h]);
    const int vx = *reinterpret_cast<const uint16_t*>(&cur.as[(rm0 + q * 32) * SCB + 2 * h]);
    f.sw[q] = LD == LD_PANEL ? vw : clean_scales(vw, st, nblk, h);
    f.sx[q] = LD == LD_PANEL ? vx : clean_scales(vx, st, nblk, h);
  }
  read_codes<0>(cur, rn0, rm0, h, f.w0, f.x0);
  read_codes<1>(cur, rn0, rm0, h, f.w1, f.x1);
}

__device__ __forceinline__ void mfma_stage(v16f acc[4][4], const Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w0[i], f.x0[j], acc[i][j], 4, 4, 0, f.sw[i], 0,
                                                                  f.sx[j]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w1[i], f.x1[j], acc[i][j], 4, 4, 1, f.sw[i], 1,
                                                                  f.sx[j]);
}

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));

// Block scale byte `B` (an E4M3 value; gfx950's FP8 is OCP E4M3FN) of a
// lane's four, as an f16 pair (s, s). The conversion is exact (E4M3 values
// are f16 values).
template <int B>
__device__ __forceinline__ h2v scale_pair(int sw) {
  constexpr uint32_t sel = (B << 24) | (B << 16) | (B << 8) | B;  // byte B into all four bytes
  const uint32_t dup = __builtin_amdgcn_perm((uint32_t)sw, (uint32_t)sw, sel);
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(dup, 1.0f, false);
}

// 8 E2M1 codes (one word, element 2p in the low nibble of byte p) times
// their block scale, as f16: the scaled convert gives the codes' values
// exactly (its scale operand is 1), and each product code x E4M3 has at
// most 6 significant bits between 2^-10 and 2688, so the f16 multiply is
// exact too.
__device__ __forceinline__ h8v dequant_nv(uint32_t w, h2v s) {
  const h2v q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const h2v q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const h2v q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const h2v q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return h8v{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
}

// NVFP4-style stage on V_MFMA_F32_32X32X16_F16. Chunk 2h + KS of lane half
// h (32 elements, 16 bytes) feeds four K steps: step ks takes its word ks
// (elements 8 ks .. 8 ks + 7, block 2 KS + ks / 2 of the lane's four), so a
// 16-element MFMA K step pairs word ks of chunk KS (lanes 0..31) with word ks
// of chunk 2 + KS (lanes 32..63) -- one K permutation, the same for both
// operands. The accumulator layout is that of the FP4 MFMA.
template <int KS>
__device__ __forceinline__ void mfma_half_nv(v16f acc[4][4], const v8i fw[4], const v8i fx[4], const int sw[4],
                                             const int sx[4]) {
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {  // the chunk's two scale blocks
    h2v swp[4], sxp[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      swp[q] = hb ? scale_pair<2 * KS + 1>(sw[q]) : scale_pair<2 * KS>(sw[q]);
      sxp[q] = hb ? scale_pair<2 * KS + 1>(sx[q]) : scale_pair<2 * KS>(sx[q]);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ks = 2 * hb + kk;
      h8v a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = dequant_nv((uint32_t)fw[q][ks], swp[q]);
        b[q] = dequant_nv((uint32_t)fx[q][ks], sxp[q]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void mfma_stage_nv(v16f acc[4][4], const Frags& f) {
  mfma_half_nv<0>(acc, f.w0, f.x0, f.sw, f.sx);
  mfma_half_nv<1>(acc, f.w1, f.x1, f.sw, f.sx);
}

// One pipeline step. On entry `cur` holds stage st's fragments (registers),
// buffer `nxt` holds or is receiving the stream's next stage, and `own` --
// the buffer stage st was read from -- is free once every wave is past this
// step's barrier. The step: wait for the next stage, barrier, start the
// stage four ahead of st into `own`, then run stage st's MFMAs while reading
// the next stage's fragments into `next`.
// (d4, st4): tile and stage of the stream element four ahead;
// st1: within-tile index of the next stage.
// after_epi: the previous tile's epilogue issued exactly EPI vector-memory
// instructions after the stages now in flight (they count in vmcnt too).
// Vector-memory instructions per wave per stage: 8 code loads plus the
// scale loads (2 words; 4 for NVFP4-style; 8 bytes through registers).
template <int LD>
constexpr int stage_vmem() { return LD == LD_NV ? 12 : (LD == LD_ROW_BYTE ? 16 : 10); }

template <int LD, int EPI = 0, bool READ_NEXT = true>
__device__ __forceinline__ void pipe_step(v16f acc[4][4], const Frags& cur, Frags& next, Stage<LD>& own,
                                          const Stage<LD>& nxt, const Problem& p, const LaneOffsets& o, const TileDesc& d4,
                                          int st4, int st1, int rn0, int rm0, int h, bool after_epi = false) {
  constexpr bool SDW = LD != LD_ROW_BYTE;
  constexpr int PER = stage_vmem<LD>();
  constexpr int ALLOW_EPI = 2 * PER + EPI < 63 ? 2 * PER + EPI : 63;
  // this wave's share of the next stage has landed; after the barrier,
  // everyone's has and nobody still reads `own`
  if (EPI > 0 && after_epi)
    wait_barrier<ALLOW_EPI>();
  else
    wait_barrier<2 * PER>();
  uint32_t sc[8];
  issue_stage<LD>(own, p, o, d4, st4, sc);
  if (READ_NEXT) read_stage<LD>(nxt, st1, p.nblk, rn0, rm0, h, next);
  if (LD == LD_NV) {
    // 128 MFMAs with the dequantization of their operands; the compiler
    // interleaves the conversions of one K step with the MFMAs of the last
    mfma_stage_nv(acc, cur);
    __builtin_amdgcn_sched_barrier(0);
    return;
  }
  mfma_stage(acc, cur);
  // schedule: MFMAs back to back, with the next stage's fragment reads and
  // the loads four stages ahead slotted between them
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
  for (int q = 0; q < 10; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 11, 0);
  __builtin_amdgcn_sched_barrier(0);
  if (!SDW) {
    // the scale bytes were issued before this stage's code loads: once only
    // those 8 remain, the bytes are in registers
    asm volatile("" ::: "memory");
    wait_vm_lgkm0<8>();
    store_scale_regs(own, sc);
  }
}

// Epilogue of one tile straight from the accumulators. For MFMA tile (i, j)
// a lane holds m = 32 j + l % 32 and n = 32 i + 8 q + 4 h + s (q, s = 0..3).
// Swapping the q = 0/1 values of the upper lane half with the q = 2/3 values
// of the lower half (v_permlane32_swap) leaves lane half h with the 16
// consecutive n 32 i + 16 h .. +15, in register order q = 0, 2, 1, 3.
__device__ __forceinline__ void gather16(v16f v, float o[16]) {
#pragma unroll
  for (int qq = 0; qq < 2; ++qq)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[4 * qq + s]),
                                                      __float_as_uint(v[4 * (qq + 2) + s]), false, false);
      v[4 * qq + s] = __uint_as_float(r[0]);
      v[4 * (qq + 2) + s] = __uint_as_float(r[1]);
    }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    o[s] = v[s];            // q = 0 slot
    o[4 + s] = v[8 + s];    // q = 2 slot
    o[8 + s] = v[4 + s];    // q = 1 slot
    o[12 + s] = v[12 + s];  // q = 3 slot
  }
}

// One accumulator, read out of its AGPR where it is used: left to itself the
// compiler copies most of the 256 accumulators to VGPRs at once at the end
// of the K loop, which leaves the GELU epilogue no registers to overlap its
// table lookups with.
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// Vector-memory instructions store_tile<FULL = true> issues per wave: per
// MFMA tile two 16-byte stores (bf16) or four (fp32), plus four residual loads.
// (RESID 2: the Euler epilogue, which also loads x; RESID 3: the GELU + MXFP4
// epilogue, 2 code stores and 1 scale store per 32 rows.)
template <int BF16OUT, int RESID>
constexpr int full_tile_vmem() {
  return (RESID == 3 || RESID == 5) ? 12
                                    : (RESID == 4 ? 16 * 12 + 5 : 16 * (BF16OUT ? 2 : (RESID == 2 ? 12 : (RESID ? 8 : 4))));
}

// MFMA tiles are stored in the order t = 4 j + i (j: m block, i: n block),
// so the two tiles i = 2k, 2k + 1 that share a 128-byte line of a bf16 row
// are written back to back.
__device__ __forceinline__ int64_t tile_offset(int t, int m_base, int n_base, int64_t ldc, int r32, int h) {
  return (int64_t)(m_base + 32 * (t >> 2) + r32) * ldc + n_base + 32 * (t & 3) + 16 * h;
}

__device__ __forceinline__ void load_res16(float4 r[4], const float* src) {
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) r[g4] = reinterpret_cast<const float4*>(src)[g4];
}

template <int BF16OUT>
__device__ __forceinline__ void store16(float o[16], void* c, int64_t off, bool rows16) {
  if (BF16OUT) {
    uint32_t wv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)  // hardware round-to-nearest-even conversion
      wv[e] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)o[2 * e], (__bf16)o[2 * e + 1]});
    if (rows16) {  // 16-byte aligned rows
      uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(c) + off);
      dst[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      dst[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
    } else {       // rows only 8-byte aligned
      uint2* dst = reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(c) + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = make_uint2(wv[2 * e], wv[2 * e + 1]);
    }
  } else {
    float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(c) + off);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) dst[g4] = make_float4(o[4 * g4], o[4 * g4 + 1], o[4 * g4 + 2], o[4 * g4 + 3]);
  }
}

// FULL: the tile lies wholly inside C and rows are 16-byte aligned, so every
// wave issues exactly full_tile_vmem() instructions and the pipeline can
// count them instead of draining them; the residual loads run two MFMA
// tiles ahead of their use (three 16-register buffers in rotation), so one
// memory round trip is exposed per tile, not one per MFMA tile. Otherwise
// element-wise tails at the N edge and the caller drains the stores.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS staging area of one wave for the epilogue of a full tile: 32 rows of
// 128 bytes (two MFMA tiles of bf16, or one of fp32), rows padded to 144
// bytes so that the accumulator-order writes and the row-order reads are
// both free of bank conflicts.
constexpr int kEpiPitch = 144;
constexpr int kEpiWaveBytes = 32 * kEpiPitch;

// Stored straight from the accumulator layout, a store instruction covers 32
// rows x two 16-byte pieces (64 scattered pieces). Instead each lane writes
// its 16 consecutive n of one row (after the lane-half swap of gather16) to
// the staging area and reads back 16 bytes of a row, so that lanes
// 8 r' .. 8 r' + 7 cover one row's 128 bytes: every store (and residual /
// state load) instruction then touches 8 whole 128-byte row segments. The
// instruction counts stay those of the direct epilogue (full_tile_vmem),
// which the pipeline's waits count.

// bf16 output: MFMA tiles (2k, j) and (2k + 1, j) share the staging area, 4
// stores per pair.
__device__ __forceinline__ void store_tile_bf16_lds(v16f acc[4][4], int m_base, int n_base, void* c, int64_t ldc,
                                                    uint8_t* stage) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));  // keep the lane-dependent address math in the epilogue, out of the K loop
  const int r32 = lane & 31, h = lane >> 5;
  const int rq = lane >> 3, cq = lane & 7;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        float o[16];
        gather16(acc[2 * k + ii][j], o);  // 16 consecutive n of row r32: 32 bytes at column byte 32 h
        uint32_t wv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)  // hardware round-to-nearest-even conversion
          wv[e] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)o[2 * e], (__bf16)o[2 * e + 1]});
        uint4* dst = reinterpret_cast<uint4*>(stage + r32 * kEpiPitch + ii * 64 + h * 32);
        dst[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        dst[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 8 * q + rq;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * kEpiPitch + cq * 16);
        // non-temporal: the output is not read again by this kernel, and the
        // L2 is left to the operand panels
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(c) +
                                                                (int64_t)(m_base + 32 * j + row) * ldc + n_base +
                                                                64 * k + 8 * cq));
      }
      __builtin_amdgcn_sched_barrier(0);  // the next pair's writes stay behind these reads
    }
}

// fp32 output, RESID 1: + residual, RESID 2: then the Euler step
// fmaf(dt, v, x) (see store_tile), RESID 4: the Euler step and the proxy
// reward's partial sum of the new state times u over the wave's 128 x 128
// values, written to *rslot. One MFMA tile at a time (t = 4 j + i), 4
// stores plus 4 residual (and 4 state) loads each; the loads run two MFMA
// tiles ahead of their use (one with the state).
template <int RESID>
__device__ __forceinline__ void store_tile_f32_lds(v16f acc[4][4], int m_base, int n_base, const Problem& p, void* c,
                                                   int64_t ldc, const float* residual, uint8_t* stage,
                                                   float* rslot = nullptr) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));  // keep the lane-dependent address math in the epilogue, out of the K loop
  const int r32 = lane & 31, h = lane >> 5;
  const int rq = lane >> 3, cq = lane & 7;
  constexpr bool EULER = RESID == 2 || RESID == 4;
  constexpr bool REWARD = RESID == 4;
  // reward: this lane's columns n_base + 32 i + 4 cq .. +3 of u, and its sum
  // over its values in (t, q) order, one fma each
  float4 uu[4];
  float racc = 0.0f;
  if (REWARD) {
#pragma unroll
    for (int i = 0; i < 4; ++i) uu[i] = *reinterpret_cast<const float4*>(p.ru + n_base + 32 * i + 4 * cq);
  }
  constexpr int LA = EULER ? 1 : 2;  // MFMA tiles of load look-ahead (registers allow one with two inputs)
  constexpr int NB = LA + 1;
  auto goff = [&](int t, int q) -> int64_t {
    return (int64_t)(m_base + 32 * (t >> 2) + 8 * q + rq) * ldc + n_base + 32 * (t & 3) + 4 * cq;
  };
  float4 rb[NB][4], xb[NB][4];
  if (RESID) {
#pragma unroll
    for (int t = 0; t < LA; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rb[t][q] = *reinterpret_cast<const float4*>(residual + goff(t, q));
        if (EULER) xb[t][q] = *reinterpret_cast<const float4*>(p.ex + goff(t, q));
      }
  }
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    if (RESID && t + LA < 16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rb[(t + LA) % NB][q] = *reinterpret_cast<const float4*>(residual + goff(t + LA, q));
        if (EULER) xb[(t + LA) % NB][q] = *reinterpret_cast<const float4*>(p.ex + goff(t + LA, q));
      }
    }
    float o16[16];
    gather16(acc[t & 3][t >> 2], o16);  // 16 consecutive n of row r32: 64 bytes at column byte 64 h
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *reinterpret_cast<float4*>(stage + r32 * kEpiPitch + h * 64 + g4 * 16) =
          make_float4(o16[4 * g4], o16[4 * g4 + 1], o16[4 * g4 + 2], o16[4 * g4 + 3]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 o = *reinterpret_cast<const float4*>(stage + (8 * q + rq) * kEpiPitch + cq * 16);
      if (RESID) {
        const float4 r = rb[t % NB][q];
        o.x += r.x; o.y += r.y; o.z += r.z; o.w += r.w;
      }
      if (EULER) {
        const float4 x = xb[t % NB][q];
        o.x = fmaf(p.dt, o.x, x.x); o.y = fmaf(p.dt, o.y, x.y); o.z = fmaf(p.dt, o.z, x.z); o.w = fmaf(p.dt, o.w, x.w);
      }
      if (REWARD) {
        const float4 w = uu[t & 3];
        racc = fmaf(o.x, w.x, racc); racc = fmaf(o.y, w.y, racc); racc = fmaf(o.z, w.z, racc);
        racc = fmaf(o.w, w.w, racc);
      }
      __builtin_nontemporal_store(f32x4{o.x, o.y, o.z, o.w}, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(c) + goff(t, q)));
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads' look-ahead, and the next writes behind these reads
  }
  if (REWARD) {
    // fixed xor tree: fp32 addition commutes, so every lane ends with the same sum
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) racc += __shfl_xor(racc, o);
    if (lane == 0) *rslot = racc;
  }
}

// Staging of one wave's codes in the GELU + MXFP4 epilogue: 32 rows of 64
// code bytes (the wave's 128 columns), 72-byte pitch (conflict-free 8-byte
// writes and 16-byte reads).
constexpr int kQPitch = 72;
constexpr int kQWaveBytes = 32 * kQPitch;

// GELU + MXFP4 quantization of a full tile's output, written in the panel
// layout for the next GEMM: z = bf16(sum) (the rounding the unfused path
// stores), g = GELU(z) from the LDS table, and each 32-block along n
// quantized by the MX rule -- the same operations as a bf16-out GEMM followed
// by fp4_quantize(z, GELU prologue, panel layout), so the same bits.
// Straight from the MFMA layout: for MFMA tile (i, j) lane (r, h) holds
// n = 32 i + 8 q + 4 h + s of row m = 32 j + r in register 4 q + s, i.e. half
// of row r's 32-block, the other half in lane (r, h ^ 1); one exchange gives
// the block amax, and each lane packs its 16 codes (bytes 4 q + 2 h and
// 4 q + 2 h + 1 of the block's 16) into two words, of which one half swap
// and two byte permutes make bytes 8 h .. 8 h + 7. The wave's 128 columns
// are one chunk of the output's panel layout (block `blk`), its 128 rows
// rows m0 .. m0 + 127 of the panel: codes of 32 rows are staged in LDS and
// leave as 2 KiB contiguous (two 16-byte stores per lane), the 4 scale bytes
// of a row as one 4-byte store.
// EXACT: GELU of the fp32 sum itself (no bf16 rounding: the table's entry
// near it and a Taylor expansion, gelu_f32_fetch / gelu_f32_finish, as in
// gelu_f32_tab_n) -- the operations of an fp32-out GEMM followed by
// fp4_quantize(GELU prologue) on its fp32 output, so the same bits.
// Quantize the 16 GELU values g of MFMA tile (i, j) (this lane's half of
// a 32-block) and stage the wave's codes; returns the block's scale byte.
// HW: the hardware converter only, with `rare` set where the block's scale
// byte S is below LO (LO >= 3 includes the ALU path's blocks, S <= 2) or
// above 252 (an infinite or NaN value): the caller redoes those with the
// exact treatment of every value and block.
template <bool HW = false, uint32_t LO = 3>
__device__ __forceinline__ uint32_t gelu_block_mx(float g[16], int i, uint8_t* stage, int r32, int h,
                                                  bool* rare = nullptr) {
  uint32_t am = amax_bits<16>(g);
  {  // the other lane half's amax: one of each swapped pair is this lane's own
    const auto sw = __builtin_amdgcn_permlane32_swap(am, am, false, false);
    am = max(sw[0], sw[1]);
  }
  const uint32_t S = mx_scale(am);
  // x: block bytes 2h, 2h+1, 4+2h, 5+2h (q = 0, 1); y: the same for q = 2, 3.
  // After the swap lane half 0 holds x of both halves, half 1 y of both.
  uint32_t x, y;
  if constexpr (HW) {
    *rare |= S - LO > 252u - LO;
    x = mx_pack8_hw(g, S);
    y = mx_pack8_hw(g + 8, S);
  } else {
    x = mx_pack8(g, S);
    y = mx_pack8(g + 8, S);
  }
  const auto xy = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  const uint32_t w0 = __builtin_amdgcn_perm(xy[1], xy[0], 0x05040100u);
  const uint32_t w1 = __builtin_amdgcn_perm(xy[1], xy[0], 0x07060302u);
  *reinterpret_cast<uint2*>(stage + r32 * kQPitch + 16 * i + 8 * h) = make_uint2(w0, w1);
  return S;
}

// Write the staged codes of 32 rows (2 KiB contiguous, two 16-byte stores per
// lane) and their 4 scale bytes per row.
__device__ __forceinline__ void gelu_rows_out(uint8_t* qc, uint8_t* qs, int m0, int j, uint32_t sreg,
                                              const uint8_t* stage, int lane, int r32, int h) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 16 * half + (lane >> 2), col = lane & 3;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * kQPitch + col * 16);
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(qc + (int64_t)(m0 + 32 * j + row) * 64 + col * 16));
  }
  if (h == 0) __builtin_nontemporal_store(sreg, reinterpret_cast<uint32_t*>(qs + (int64_t)(m0 + 32 * j + r32) * 4));
  __builtin_amdgcn_sched_barrier(0);  // the next rows' staging writes stay behind these reads
}

// The wave's 16 MFMA tiles as one compile-time sequence (compile-time tile
// indices keep the accumulators in registers; an (i, j) loop around the
// erfc fallback's loop stayed rolled, indexing them at run time), with the
// table reads of the next 16 values in flight while the current ones are
// evaluated and quantized. FAST: no branches, `rare` as described where this
// is called; otherwise the exact treatment of every value and block.
template <bool FAST>
__device__ __forceinline__ void gelu_tile_f32(v16f acc[4][4], uint8_t* qc, uint8_t* qs, int m0, uint8_t* stage,
                                              const float2* tab2, bool* rare) {
  // each pass forms its own lane-dependent addresses, so that none is held
  // from the first pass through the second
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int r32 = lane & 31, h = lane >> 5;
  GeluBatch<16> cur;
#pragma unroll
  for (int e = 0; e < 16; ++e) cur.z[e] = acc_read(acc[0][0][e]);
  gelu_f32_fetch<16, !FAST>(cur, tab2);
  uint32_t sreg = 0;
  static_for<0, 16>([&](auto gc) {
    constexpr int G = decltype(gc)::value, j = G / 4, i = G % 4;
    auto finish = [&](const GeluBatch<16>& b) {
      float g[16];
      if constexpr (FAST) {
        gelu_f32_expand(g, b);
        sreg |= gelu_block_mx<true, 103>(g, i, stage, r32, h, rare) << (8 * i);
      } else {
        gelu_f32_finish(g, b);
        sreg |= gelu_block_mx(g, i, stage, r32, h) << (8 * i);
      }
      if constexpr (i == 3) {
        gelu_rows_out(qc, qs, m0, j, sreg, stage, lane, r32, h);
        sreg = 0;
      }
    };
    if constexpr (G + 1 < 16) {
      GeluBatch<16> nxt;
#pragma unroll
      for (int e = 0; e < 16; ++e) nxt.z[e] = acc_read(acc[(G + 1) % 4][(G + 1) / 4][e]);
      gelu_f32_fetch<16, !FAST>(nxt, tab2);
      finish(cur);
      cur = nxt;
    } else {
      finish(cur);
    }
  });
}

// The bf16 reading: GELU of bf16(sum) from the LDS table of Q, exact for
// every value, so only the converter differs between the passes. FAST: the
// hardware converter for every block, `rare` set where a block's scale byte
// is 2 or less (or above 252, which changes nothing but is cheap to test).
template <bool FAST>
__device__ __forceinline__ void gelu_tile_bf16(v16f acc[4][4], uint8_t* qc, uint8_t* qs, int m0, uint8_t* stage,
                                               const float* tab, bool* rare) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t sreg = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float g[16];
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // hardware round-to-nearest-even bf16 of n-adjacent pairs, back to fp32 exactly
        const float a0 = acc_read(acc[i][j][2 * e]), a1 = acc_read(acc[i][j][2 * e + 1]);
        uint32_t u = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a0, (__bf16)a1});
        asm("" : "+v"(u));  // one pair conversion (the compiler would convert the even element again on its own)
        g[2 * e] = __uint_as_float(u << 16);
        g[2 * e + 1] = __uint_as_float(u & 0xFFFF0000u);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) g[e] = gelu_bf16(g[e], tab);
      if constexpr (FAST)
        sreg |= gelu_block_mx<true, 3>(g, i, stage, r32, h, rare) << (8 * i);
      else
        sreg |= gelu_block_mx(g, i, stage, r32, h) << (8 * i);
    }
    gelu_rows_out(qc, qs, m0, j, sreg, stage, lane, r32, h);
  }
}

template <bool EXACT>
__device__ __forceinline__ void store_tile_gelu_mx(v16f acc[4][4], int64_t blk, int m0, const Problem& p,
                                                   uint8_t* stage, const float* tab, const float2* tab2) {
  // (each pass forms its lane-dependent addresses itself, behind an asm
  // barrier that keeps that arithmetic out of the K loop)
  uint8_t* qc = p.qc + blk * 16384;
  uint8_t* qs = p.qs + blk * 1024;
  if constexpr (EXACT) {
    // First a pass with no branch in it: the expansion for every value (no
    // erfc beyond |z| = 6) and the hardware converter for every block. Its
    // codes and scales are the exact ones unless some block's scale byte S
    // is below 103 or above 252:
    //   * for z > 6 both treatments give z, so those values agree;
    //   * for z < -6 both give a negative value below 6e-9 or -0, and where
    //     S >= 103 the block's amax is at least 2^-22 (set by a value that
    //     both treatments share) and its scale at least 2^-24, so both
    //     round to the negative zero code;
    //   * NaN, infinite and overflowing values make the block's S 253.
    // Such blocks do not occur in practice; where one does, somewhere in the
    // wave's tile, the wave writes the whole tile again with the exact
    // treatment (the same addresses from the same lanes, in program order,
    // so the second writes are the ones that stay). A branch inside the
    // pass would end the scheduler's region at every 16 values; without
    // them the pass runs about 20% faster.
    bool rare = false;
    gelu_tile_f32<true>(acc, qc, qs, m0, stage, tab2, &rare);
    if (__any(rare)) {
      // a compiler memory barrier: nothing the first pass loaded is kept for
      // the second, which would hold the whole tile's table entries at once
      asm volatile("" ::: "memory");
      gelu_tile_f32<false>(acc, qc, qs, m0, stage, tab2, nullptr);
    }
  } else {
    // the same two passes for the bf16 reading (only the converter's
    // branch is at stake there)
    bool rare = false;
    gelu_tile_bf16<true>(acc, qc, qs, m0, stage, tab, &rare);
    if (__any(rare)) {
      asm volatile("" ::: "memory");
      gelu_tile_bf16<false>(acc, qc, qs, m0, stage, tab, nullptr);
    }
  }
}

// SCALE: multiply the sums by `mul` (the NVFP4-style tensor scales) before
// the residual is added.
// RESID 2 (the Euler epilogue, fp32 out): v = fl(sum + residual), then
// C = fmaf(dt, v, x) with x = p.ex and dt = p.dt -- the operations of a
// residual GEMM into v followed by the Euler kernel, so bit-identical to
// them. Every element is read and written by the same lane, so C may alias
// x or residual.
// v = sum * scale + residual for four values, the tensor-scale product fused
// into the add (one rounding; with no tensor scale, scale is 1 and this is
// the plain add). Written out so that every epilogue path rounds alike.
__device__ __forceinline__ void scale_add(float* o, float mt, float4 r) {
  o[0] = fmaf(o[0], mt, r.x); o[1] = fmaf(o[1], mt, r.y); o[2] = fmaf(o[2], mt, r.z); o[3] = fmaf(o[3], mt, r.w);
}

// NVFP4-style: the product of the two tensor scales for output row m -- one
// for the whole call, or A's scale of m's row group times B's.
__device__ __forceinline__ float row_scale(const Problem& p, int m, float mul) {
  if (p.a_rpg == 0) return mul;
  const int mc = m < p.M ? m : p.M - 1;
  return p.a_ts[(uint32_t)mc / (uint32_t)p.a_rpg] * (*p.b_ts);
}

template <int BF16OUT, int RESID, bool FULL, bool SCALE>
__device__ __forceinline__ void store_tile(v16f acc[4][4], int m_base, int n_base, const Problem& p, void* c,
                                           int64_t ldc, const float* residual, float mul) {
  const int lane = threadIdx.x & 63, r32 = lane & 31, h = lane >> 5;
  constexpr bool EULER = RESID == 2;
  if (FULL) {
    float4 rq[3][4], xq[3][4];
    if (RESID) {
      load_res16(rq[0], residual + tile_offset(0, m_base, n_base, ldc, r32, h));
      if (EULER) load_res16(xq[0], p.ex + tile_offset(0, m_base, n_base, ldc, r32, h));
      load_res16(rq[1], residual + tile_offset(1, m_base, n_base, ldc, r32, h));
      if (EULER) load_res16(xq[1], p.ex + tile_offset(1, m_base, n_base, ldc, r32, h));
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (RESID && t + 2 < 16) {
        load_res16(rq[(t + 2) % 3], residual + tile_offset(t + 2, m_base, n_base, ldc, r32, h));
        if (EULER) load_res16(xq[(t + 2) % 3], p.ex + tile_offset(t + 2, m_base, n_base, ldc, r32, h));
      }
      float o[16];
      gather16(acc[t & 3][t >> 2], o);
      const float mt = SCALE ? row_scale(p, m_base + 32 * (t >> 2) + r32, mul) : 1.0f;
      if (RESID) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 r4 = rq[t % 3][g4];
          scale_add(o + 4 * g4, mt, r4);
        }
      } else if (SCALE) {
#pragma unroll
        for (int e = 0; e < 16; ++e) o[e] *= mt;
      }
      if (EULER) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 x4 = xq[t % 3][g4];
          o[4 * g4] = fmaf(p.dt, o[4 * g4], x4.x); o[4 * g4 + 1] = fmaf(p.dt, o[4 * g4 + 1], x4.y);
          o[4 * g4 + 2] = fmaf(p.dt, o[4 * g4 + 2], x4.z); o[4 * g4 + 3] = fmaf(p.dt, o[4 * g4 + 3], x4.w);
        }
      }
      store16<BF16OUT>(o, c, tile_offset(t, m_base, n_base, ldc, r32, h), true);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads' look-ahead at two tiles
    }
    return;
  }
  const bool rows16 = BF16OUT ? (ldc & 7) == 0 : true;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    float o[16];
    gather16(acc[t & 3][t >> 2], o);
    const int m = m_base + 32 * (t >> 2) + r32;
    const float mt = SCALE ? row_scale(p, m, mul) : 1.0f;
    if (SCALE && !RESID) {
#pragma unroll
      for (int e = 0; e < 16; ++e) o[e] *= mt;
    }
    const int n = n_base + 32 * (t & 3) + 16 * h;
    if (m >= p.M || n >= p.N) continue;
    const int64_t off = (int64_t)m * ldc + n;
    if (n + 16 <= p.N) {
      if (RESID) {
        float4 r[4];
        load_res16(r, residual + off);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) scale_add(o + 4 * g4, mt, r[g4]);
      }
      if (EULER) {
        float4 x4[4];
        load_res16(x4, p.ex + off);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          o[4 * g4] = fmaf(p.dt, o[4 * g4], x4[g4].x); o[4 * g4 + 1] = fmaf(p.dt, o[4 * g4 + 1], x4[g4].y);
          o[4 * g4 + 2] = fmaf(p.dt, o[4 * g4 + 2], x4[g4].z); o[4 * g4 + 3] = fmaf(p.dt, o[4 * g4 + 3], x4[g4].w);
        }
      }
      store16<BF16OUT>(o, c, off, rows16);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (n + e >= p.N) continue;
        float x = o[e];
        if (RESID) x = fmaf(x, mt, residual[off + e]);
        if (EULER) x = fmaf(p.dt, x, p.ex[off + e]);
        if (BF16OUT)
          reinterpret_cast<__bf16*>(c)[off + e] = (__bf16)x;
        else
          reinterpret_cast<float*>(c)[off + e] = x;
      }
    }
  }
}

// The persistent GEMM of either format: LD_ROW_BYTE, LD_ROW_WORD and
// LD_PANEL take MXFP4 operands, LD_NV NVFP4-style ones. (One kernel body
// for all: wrapping it in a device function made the compiler spill.)
template <int BF16OUT, int RESID, int LD>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp4_kernel(Problem p, void* __restrict__ c, int64_t ldc,
                                                               const float* residual, int nst4) {
  constexpr int EPI = full_tile_vmem<BF16OUT, RESID>();
  constexpr bool NV = LD == LD_NV;
  const bool rows16 = BF16OUT ? (ldc % 8 == 0) : true;  // 16-byte aligned output rows
  __shared__ Stage<LD> s0, s1, s2, s3;
  // full tiles' epilogue through an LDS staging area (the MXFP4 ring leaves
  // room for it; the NVFP4-style ring, with twice the scale bytes, does not);
  // the GELU + MXFP4 epilogue has its own, smaller one and the GELU table
  constexpr bool GELU_Q = RESID == 3 || RESID == 5;  // 5: GELU of the fp32 sum, 3: of its bf16 rounding
  constexpr bool EPI_LDS = !NV && !GELU_Q;
  // The GELU + MXFP4 epilogue needs the registers that the next tile's first
  // fragments would hold across it: it reads them afterwards.
  constexpr bool DEFER_READ = GELU_Q;
  __shared__ __attribute__((aligned(16))) uint8_t epi_stage[EPI_LDS ? 4 * kEpiWaveBytes : (GELU_Q ? 4 * kQWaveBytes : 16)];
  // GELU tables, visible to all waves after the first pipeline barrier
  __shared__ float gtab[RESID == 3 ? kGeluTab : 1];     // bf16 sums: Q at every bf16 magnitude from 2^-22
  __shared__ float2 gtab2[RESID == 5 ? kGeluTTab : 1];  // fp32 sums: (Q, phi) from 2^-10, Taylor in between
  if (RESID == 3) gelu_table_fill(gtab);
  if (RESID == 5) gelu_table_fill(gtab2);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // the wave's 128 x 128 sub-tile
  const int r32 = lane & 31, h = lane >> 5;
  const int rn0 = wn * 128 + r32, rm0 = wm * 128 + r32;
  const int G = gridDim.x, g = blockIdx.x;
  if (g >= p.total) return;

  constexpr bool SDW = LD != LD_ROW_BYTE;
  LaneOffsets o;
  make_lane_offsets<LD>(o, p);

  // Prologue: the stream's first four stages (tile g, stages 0..3; nst4 >= 4).
  // The stage waits count this wave's loads in issue order, so no load may
  // move across a stage boundary.
  TileDesc dcur = make_desc<LD>(p, g);
  {
    uint32_t sc[8];
    issue_stage<LD>(s0, p, o, dcur, 0, sc);
    asm volatile("" ::: "memory");
    if (!SDW) { wait_vm_lgkm0<8>(); store_scale_regs(s0, sc); }
    issue_stage<LD>(s1, p, o, dcur, 1, sc);
    asm volatile("" ::: "memory");
    if (!SDW) { wait_vm_lgkm0<8>(); store_scale_regs(s1, sc); }
    issue_stage<LD>(s2, p, o, dcur, 2, sc);
    asm volatile("" ::: "memory");
    if (!SDW) { wait_vm_lgkm0<8>(); store_scale_regs(s2, sc); }
    issue_stage<LD>(s3, p, o, dcur, 3, sc);
    asm volatile("" ::: "memory");
    if (!SDW) { wait_vm_lgkm0<8>(); store_scale_regs(s3, sc); }
  }
  constexpr int PER = stage_vmem<LD>();
  wait_barrier<3 * PER>();  // stage 0 has landed (this wave's share, then everyone's)
  const float mul = NV ? (*p.a_ts) * (*p.b_ts) : 1.0f;
  Frags fa, fb;
  read_stage<LD>(s0, 0, p.nblk, rn0, rm0, h, fa);

  bool counted = false;  // the previous tile's stores are counted, not drained
  for (int pid = g; pid < p.total; pid += G) {
    int tm, tn;
    tile_coords(pid, p.tiles_m, p.tiles_n, tm, tn);
    const TileDesc dnext = make_desc<LD>(p, pid + G);
    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
    // The per-tile stage count nst4 is a multiple of 4 (the ring size); the
    // stages past K hold only zero codes and add nothing. In the last group
    // the stages four ahead belong to the next tile.
    for (int st = 0; st < nst4; st += NBUF) {
      const bool last = st + NBUF == nst4;
      const TileDesc& d4 = last ? dnext : dcur;
      const int b4 = last ? 0 : st + NBUF;
      pipe_step<LD, EPI>(acc, fa, fb, s0, s1, p, o, d4, b4, st + 1, rn0, rm0, h, counted && st == 0);
      pipe_step<LD>(acc, fb, fa, s1, s2, p, o, d4, b4 + 1, st + 2, rn0, rm0, h);
      pipe_step<LD>(acc, fa, fb, s2, s3, p, o, d4, b4 + 2, st + 3, rn0, rm0, h);
      pipe_step<LD>(acc, fb, fa, s3, s0, p, o, d4, b4 + 3, last ? 0 : st + 4, rn0, rm0, h);
    }
    dcur = dnext;
    int mb = tm * BM + wm * 128, nb = tn * BN + wn * 128;
    asm volatile("" : "+v"(mb), "+v"(nb));  // keep epilogue address math out of the main loop
    counted = rows16 && (tm + 1) * BM <= p.M && (tn + 1) * BN <= p.N;
    if (GELU_Q) {
      // every tile is full (the host launches this epilogue only for m, n multiples of 256)
      store_tile_gelu_mx<RESID == 5>(acc, (int64_t)tm * p.qnc + 2 * tn + wn, wm * 128, p,
                                     epi_stage + wave * kQWaveBytes, gtab, gtab2);
      counted = true;
    } else if (counted) {
      if (EPI_LDS && BF16OUT)
        store_tile_bf16_lds(acc, mb, nb, c, ldc, epi_stage + wave * kEpiWaveBytes);
      else if (EPI_LDS)
        store_tile_f32_lds<RESID>(acc, mb, nb, p, c, ldc, residual, epi_stage + wave * kEpiWaveBytes,
                                  RESID == 4 ? p.rp + ((int64_t)tm * p.tiles_n + tn) * 4 + wave : nullptr);
      else
        store_tile<BF16OUT, RESID, true, NV>(acc, mb, nb, p, c, ldc, residual, mul);
    } else {
      store_tile<BF16OUT, RESID, false, NV>(acc, mb, nb, p, c, ldc, residual, mul);
      __builtin_amdgcn_s_waitcnt(0);  // an edge tile's stores are not counted: drain them here
    }
    // DEFER_READ: the next tile's first fragments, read by the last step,
    // are read again here, so that they need no registers during the
    // epilogue. Buffer s0 holds that stage (landed: the last step waited for
    // it) until every wave has passed the next step's barrier.
    if (DEFER_READ) read_stage<LD>(s0, 0, p.nblk, rn0, rm0, h, fa);
  }
  __builtin_amdgcn_s_waitcnt(0);  // drain the trailing (past-the-end) loads before the workgroup exits
}


// CUs of the device current at the first call (thread-safe static
// initialization; the library runs on one kind of GPU): the persistent grid.
int cu_count() {
  static const int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                 hipSuccess && v > 0)
      return v;
    return 256;
  }();
  return n;
}

template <int BF16OUT, int RESID>
hipError_t launch(const Problem& p, void* c, int64_t ldc, const float* residual, hipStream_t st, int ld) {
  const int nst4 = (p.nkc + NBUF - 1) / NBUF * NBUF;
  const unsigned grid = (unsigned)min(p.total, cu_count());
  if (ld == LD_NV)
    gemm_fp4_kernel<BF16OUT, RESID, LD_NV><<<grid, kThreads, 0, st>>>(p, c, ldc, residual, nst4);
  else if (ld == LD_PANEL)
    gemm_fp4_kernel<BF16OUT, RESID, LD_PANEL><<<grid, kThreads, 0, st>>>(p, c, ldc, residual, nst4);
  else if (ld == LD_ROW_WORD)
    gemm_fp4_kernel<BF16OUT, RESID, LD_ROW_WORD><<<grid, kThreads, 0, st>>>(p, c, ldc, residual, nst4);
  else
    gemm_fp4_kernel<BF16OUT, RESID, LD_ROW_BYTE><<<grid, kThreads, 0, st>>>(p, c, ldc, residual, nst4);
  return hipGetLastError();
}

hipError_t dispatch(const Problem& p, void* c, int c_bf16, int64_t ldc, const float* residual, hipStream_t st, int ld) {
  if (c_bf16) return launch<1, 0>(p, c, ldc, nullptr, st, ld);
  if (residual) return launch<0, 1>(p, c, ldc, residual, st, ld);
  return launch<0, 0>(p, c, ldc, nullptr, st, ld);
}

Problem make_problem(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs, int64_t m, int64_t n,
                     int64_t k) {
  Problem p;
  p.a = a; p.as = as; p.b = b; p.bs = bs;
  p.a_ts = p.b_ts = nullptr;
  p.a_rpg = 0;
  p.ex = nullptr;
  p.dt = 0.0f;
  p.qc = p.qs = nullptr;
  p.qnc = 0;
  p.ru = nullptr;
  p.rp = nullptr;
  p.lda = p.ld_as = p.ldb = p.ld_bs = 0;
  p.M = (int)m; p.N = (int)n; p.kbytes = (int)(k >> 1); p.nblk = (int)(k >> 5);
  p.nkc = (int)((k + 127) >> 7);
  p.tiles_m = (int)((m + BM - 1) / BM); p.tiles_n = (int)((n + BN - 1) / BN);
  p.total = p.tiles_m * p.tiles_n;
  return p;
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as, const uint8_t* b,
                          int64_t ldb, const uint8_t* bs, int64_t ld_bs, int64_t m, int64_t n, int64_t k, void* c,
                          int c_bf16, int64_t ldc, const float* residual, hipStream_t st) {
  Problem p = make_problem(a, as, b, bs, m, n, k);
  p.lda = lda; p.ld_as = ld_as; p.ldb = ldb; p.ld_bs = ld_bs;
  // scales as whole 4-byte words when every row's scale bytes start 4-byte aligned
  const bool sdw = (ld_as % 4 == 0) && (ld_bs % 4 == 0) && (reinterpret_cast<uintptr_t>(as) % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(bs) % 4 == 0);
  return dispatch(p, c, c_bf16, ldc, residual, st, sdw ? LD_ROW_WORD : LD_ROW_BYTE);
}

// NVFP4-style operands with 4-byte aligned scale rows (16 scale bytes per
// 256 K-elements, 8 per stage).
hipError_t launch_gemm_nv_f16(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as, const float* a_ts,
                              const uint8_t* b, int64_t ldb, const uint8_t* bs, int64_t ld_bs, const float* b_ts,
                              int64_t m, int64_t n, int64_t k, void* c, int c_bf16, int64_t ldc, const float* residual,
                              hipStream_t st, int64_t a_rows_per_group) {
  Problem p = make_problem(a, as, b, bs, m, n, k);
  p.lda = lda; p.ld_as = ld_as; p.ldb = ldb; p.ld_bs = ld_bs;
  p.nblk = (int)(k >> 4);
  p.a_ts = a_ts; p.b_ts = b_ts;
  p.a_rpg = (int)a_rows_per_group;
  return dispatch(p, c, c_bf16, ldc, residual, st, LD_NV);
}

// The last velocity block fused with the Euler step: x_out = x + dt (residual
// + A_hat B_hat^T), MXFP4 panel operands, fp32 [m, ldx] state.
hipError_t launch_gemm_mx_panel_euler(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                                      int64_t m, int64_t n, int64_t k, const float* residual, const float* x,
                                      float* x_out, int64_t ldx, float dt, hipStream_t st) {
  Problem p = make_problem(a, as, b, bs, m, n, k);
  p.ex = x;
  p.dt = dt;
  const int nst4 = (p.nkc + NBUF - 1) / NBUF * NBUF;
  const unsigned grid = (unsigned)min(p.total, cu_count());
  gemm_fp4_kernel<0, 2, LD_PANEL><<<grid, kThreads, 0, st>>>(p, x_out, ldx, residual, nst4);
  return hipGetLastError();
}

// The proxy reward of each candidate from the Euler + reward epilogue's
// per-wave partial sums: candidate c owns the waves whose 128 rows lie in its
// rows_per_cand rows (wave w of tile (tm, tn) covers rows tm 256 + 128 (w & 1)
// ..., columns tn 256 + 128 (w >> 1) ...). Sum in a fixed order (per thread,
// then a fixed shuffle tree and LDS order), divided by rows_per_cand.
namespace {
__global__ __launch_bounds__(256) void reward_partials_kernel(const float* __restrict__ rp, int tiles_n,
                                                              int rows_per_cand, float* __restrict__ rewards) {
  __shared__ float sh[4];
  const int c = blockIdx.x;
  const int wrows = rows_per_cand / 128;  // wave rows per candidate
  const int per_wr = tiles_n * 2;         // partials per wave row: every tile column, both column halves
  const int total = wrows * per_wr;
  float acc = 0.0f;
  for (int f = threadIdx.x; f < total; f += 256) {
    const int wr = c * wrows + f / per_wr;  // global wave row: tm = wr / 2, row half wr % 2
    const int tn = (f % per_wr) >> 1, wn = f & 1;
    acc += rp[((int64_t)(wr >> 1) * tiles_n + tn) * 4 + (wr & 1) + 2 * wn];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) rewards[c] = (((sh[0] + sh[1]) + sh[2]) + sh[3]) / (float)rows_per_cand;
}
}  // namespace

// The last block of the last Euler step with the proxy reward in the same
// pass: x_out as launch_gemm_mx_panel_euler, then rewards[c] = mean over the
// candidate's rows of <x_out row, u>. m and n are multiples of 256 and
// rows_per_cand of 128, dividing m (checked by the caller); partials holds
// (m / 256) (n / 256) 4 floats.
hipError_t launch_gemm_mx_panel_euler_reward(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                                             int64_t m, int64_t n, int64_t k, const float* residual, const float* x,
                                             float* x_out, int64_t ldx, float dt, const float* u, int64_t rows_per_cand,
                                             float* partials, float* rewards, hipStream_t st) {
  Problem p = make_problem(a, as, b, bs, m, n, k);
  p.ex = x;
  p.dt = dt;
  p.ru = u;
  p.rp = partials;
  const int nst4 = (p.nkc + NBUF - 1) / NBUF * NBUF;
  const unsigned grid = (unsigned)min(p.total, cu_count());
  gemm_fp4_kernel<0, 4, LD_PANEL><<<grid, kThreads, 0, st>>>(p, x_out, ldx, residual, nst4);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  reward_partials_kernel<<<(unsigned)(m / rows_per_cand), 256, 0, st>>>(partials, p.tiles_n, (int)rows_per_cand,
                                                                        rewards);
  return hipGetLastError();
}

// Scratch for fp4_gemm_panel_euler_reward_noalloc: the per-wave partial sums
// of the Euler + reward epilogue, for callers that cannot allocate (graph
// capture, serving loops). One copy per GPU, held until the process ends. In
// host code `scratch` names a host-side stand-in, not the device array: its
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[kNoAllocPartials];

hipError_t noalloc_partials(float** ptr) {
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// launch_gemm_mx_panel_euler_reward with the partial sums in `scratch`; the
// caller has checked (m / 256) (n / 256) 4 <= kNoAllocPartials. Every partial
// is written by the GEMM before the reward kernel reads it, so nothing needs
// clearing between calls.
hipError_t launch_gemm_mx_panel_euler_reward_noalloc(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                                                     const uint8_t* bs, int64_t m, int64_t n, int64_t k,
                                                     const float* residual, const float* x, float* x_out, int64_t ldx,
                                                     float dt, const float* u, int64_t rows_per_cand, float* rewards,
                                                     hipStream_t st) {
  float* part = nullptr;
  const hipError_t e = noalloc_partials(&part);
  if (e != hipSuccess) return e;
  return launch_gemm_mx_panel_euler_reward(a, as, b, bs, m, n, k, residual, x, x_out, ldx, dt, u, rows_per_cand, part,
                                           rewards, st);
}

// The first solver linear with GELU and MXFP4 quantization of its output in
// its epilogue: codes / scales of GELU(bf16(A_hat B_hat^T)) in the panel
// layout of an [m, n] operand -- or, with `exact`, of GELU of the fp32 sums
// themselves. m and n must be multiples of 256 (checked by the caller).
hipError_t launch_gemm_mx_panel_gelu(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                                     int64_t m, int64_t n, int64_t k, uint8_t* out_codes, uint8_t* out_scales,
                                     int exact, hipStream_t st) {
  Problem p = make_problem(a, as, b, bs, m, n, k);
  p.qc = out_codes;
  p.qs = out_scales;
  p.qnc = (int)(n / 128);
  const int nst4 = (p.nkc + NBUF - 1) / NBUF * NBUF;
  const unsigned grid = (unsigned)min(p.total, cu_count());
  if (exact)
    gemm_fp4_kernel<0, 5, LD_PANEL><<<grid, kThreads, 0, st>>>(p, nullptr, 0, nullptr, nst4);
  else
    gemm_fp4_kernel<0, 3, LD_PANEL><<<grid, kThreads, 0, st>>>(p, nullptr, 0, nullptr, nst4);
  return hipGetLastError();
}

hipError_t launch_gemm_mx_panel(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs, int64_t m,
                                int64_t n, int64_t k, void* c, int c_bf16, int64_t ldc, const float* residual,
                                hipStream_t st) {
  return dispatch(make_problem(a, as, b, bs, m, n, k), c, c_bf16, ldc, residual, st, LD_PANEL);
}

}  // namespace fp4r
