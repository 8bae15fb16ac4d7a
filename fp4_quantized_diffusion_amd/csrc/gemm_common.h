// Tile loading and epilogue helpers shared by the FP4 GEMM kernels (gfx950).
//
// Both GEMMs stage 256 x 256 output tiles with 256-element K stages held in
// LDS; codes are row-major packed nibbles (16-byte chunks), scales one byte
// per K-block. Global reads go through buffer resources, whose out-of-range
// reads return zero: rows past M / N and K past the end need no branches.
#pragma once
#include "common.h"

namespace fp4r {
namespace gemm {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256;
constexpr int BKB = 128;            // bytes of codes per row per stage (256 elements)
constexpr int ROWB = BKB + 16;      // padded LDS row stride (bank-conflict padding)
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

// Workgroup -> output tile. Dispatch hands consecutive workgroups to the 8
// XCDs in turn; renumber so that XCD x owns a contiguous range of tiles, and
// walk that range in groups of kGroupM tile-rows so tiles running together
// on one XCD share A and B panels in its L2.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int xcd = pid % kXcds, j = pid / kXcds;
  const int base = total / kXcds, rem = total % kXcds;
  const int logical = xcd * base + min(xcd, rem) + j;
  const int per_group = kGroupM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Buffer resource over [base, base + bytes): loads past the end return zero.
// Word 3 = 0x00020000 selects 32-bit raw (untyped) access on gfx9.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFFFll ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

constexpr uint32_t kOob = 0x7FFFFFF0u;  // an offset past every resource's end

struct Operand {
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t off[8];   // this thread's 8 rows (it * 32 + t / 8), chunk t % 8
  uint32_t soff;     // this thread's scale row t
};

__device__ __forceinline__ void make_operand(Operand& o, const uint8_t* codes, int64_t ld, const uint8_t* scales,
                                             int64_t ld_s, int row0, int rows) {
  const int valid = min(rows - row0, 256);
  o.codes = make_rsrc(codes + (int64_t)row0 * ld, (int64_t)valid * ld);
  o.scales = make_rsrc(scales + (int64_t)row0 * ld_s, (int64_t)valid * ld_s);
  const int t = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 8; ++it) o.off[it] = (uint32_t)((it * 32 + (t >> 3)) * ld + (t & 7) * 16);
  o.soff = (uint32_t)(t * ld_s);
}

// Global -> registers for one stage starting at code byte `kb`. Chunks at or
// past `kbytes` (the row's code length) read as zero codes; their scale
// bytes read as zero too, and zero codes contribute nothing whatever the
// scale. SB = scale bytes per row per stage (8: MX, 16: NV); `bpb` = code
// bytes per scale block (16: MX, 8: NV).
template <int SB>
__device__ __forceinline__ void load_operand(uint4 q[8], uint32_t sc[SB], const Operand& o, int kb, int kbytes,
                                             int bpb) {
  const int chunk = threadIdx.x & 7;
  const bool kin = kb + chunk * 16 < kbytes;
#pragma unroll
  for (int it = 0; it < 8; ++it)
    q[it] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(o.codes, kin ? o.off[it] : kOob, kb, 0));
  // scale bytes stay unpacked until the stage is stored to LDS, so no wait on
  // them is needed before the MFMAs that overlap these loads
  const int kblk = kb / bpb, nblk = kbytes / bpb;
#pragma unroll
  for (int j = 0; j < SB; ++j)
    sc[j] = __builtin_amdgcn_raw_buffer_load_b8(o.scales, kblk + j < nblk ? o.soff + j : kOob, kblk, 0);
}

template <int SB>
struct Smem {
  uint8_t a[2][BM * ROWB];
  uint8_t b[2][BN * ROWB];
  uint8_t as[2][BM * SB];
  uint8_t bs[2][BN * SB];
};

template <int SB>
struct Prefetch {
  uint4 a[8], b[8];
  uint32_t as[SB], bs[SB];  // one scale byte per register
};

template <int SB>
__device__ __forceinline__ void load_stage(Prefetch<SB>& p, const Operand& oa, const Operand& ob, int kb, int kbytes,
                                           int bpb) {
  load_operand<SB>(p.a, p.as, oa, kb, kbytes, bpb);
  load_operand<SB>(p.b, p.bs, ob, kb, kbytes, bpb);
}

template <int SB>
__device__ __forceinline__ void store_stage(Smem<SB>& s, int buf, const Prefetch<SB>& p) {
  const int t = threadIdx.x;
  const int chunk = t & 7;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = it * 32 + (t >> 3);
    *reinterpret_cast<uint4*>(&s.a[buf][r * ROWB + chunk * 16]) = p.a[it];
    *reinterpret_cast<uint4*>(&s.b[buf][r * ROWB + chunk * 16]) = p.b[it];
  }
  uint32_t wa[SB / 4], wb[SB / 4];
#pragma unroll
  for (int w = 0; w < SB / 4; ++w) {
    wa[w] = p.as[4 * w] | (p.as[4 * w + 1] << 8) | (p.as[4 * w + 2] << 16) | (p.as[4 * w + 3] << 24);
    wb[w] = p.bs[4 * w] | (p.bs[4 * w + 1] << 8) | (p.bs[4 * w + 2] << 16) | (p.bs[4 * w + 3] << 24);
  }
  if (SB == 8) {
    *reinterpret_cast<uint2*>(&s.as[buf][t * SB]) = make_uint2(wa[0], wa[1]);
    *reinterpret_cast<uint2*>(&s.bs[buf][t * SB]) = make_uint2(wb[0], wb[1]);
  } else {
    *reinterpret_cast<uint4*>(&s.as[buf][t * SB]) = make_uint4(wa[0], wa[1], wa[2 % (SB / 4)], wa[3 % (SB / 4)]);
    *reinterpret_cast<uint4*>(&s.bs[buf][t * SB]) = make_uint4(wb[0], wb[1], wb[2 % (SB / 4)], wb[3 % (SB / 4)]);
  }
}

// Epilogue store of a 16 x 16 accumulator tile held as D[n = 4g + j][m = r16]:
// lane writes C[m][n .. n+3] (+ residual), scaled by `mul`.
template <int BF16OUT, int RESID>
__device__ __forceinline__ void store_acc(v4f v, int m, int n, int M, int N, void* __restrict__ c, int64_t ldc,
                                          const float* residual, float mul) {
  if (m >= M || n >= N) return;
  v[0] *= mul; v[1] *= mul; v[2] *= mul; v[3] *= mul;
  const int64_t off = (int64_t)m * ldc + n;
  if (n + 4 <= N) {
    if (RESID) {
      const float4 r = *reinterpret_cast<const float4*>(residual + off);
      v[0] += r.x; v[1] += r.y; v[2] += r.z; v[3] += r.w;
    }
    if (BF16OUT) {
      uint2 q;
      q.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
      q.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(c) + off) = q;
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(c) + off) = make_float4(v[0], v[1], v[2], v[3]);
    }
  } else {
    for (int q = 0; q < 4 && n + q < N; ++q) {
      float o = v[q];
      if (RESID) o += residual[off + q];
      if (BF16OUT)
        reinterpret_cast<uint16_t*>(c)[off + q] = f32_to_bf16(o);
      else
        reinterpret_cast<float*>(c)[off + q] = o;
    }
  }
}

}  // namespace gemm
}  // namespace fp4r
