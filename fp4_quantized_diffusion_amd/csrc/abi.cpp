// C ABI of the fp4rollout library: argument validation and dispatch.
//
// Plain host C++ (built with the host compiler against the HIP runtime
// headers). Every check runs before anything is enqueued, so an invalid call
// launches nothing and touches no output; no C++ exception crosses the ABI.
#include "fp4rollout.h"

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <exception>

#include "common_host.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // rows, k, ld* upper bound (exclusive)

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

fp4_status from_hip(hipError_t e) { return e == hipSuccess ? FP4_OK : FP4_DEVICE_ERROR; }

fp4_status check_quantize(int fmt, const void* x, int x_dtype, int64_t rows, int64_t k, int64_t ldx,
                          const uint8_t* codes, int64_t ld_codes, const uint8_t* scales, int64_t ld_scales,
                          const float* tensor_scale, int flags) {
  if (fmt != FP4_FMT_MX && fmt != FP4_FMT_NV) return FP4_INVALID_ARGUMENT;
  if (!x || !codes || !scales) return FP4_INVALID_ARGUMENT;
  if (x_dtype != FP4_DT_F32 && x_dtype != FP4_DT_BF16) return FP4_INVALID_ARGUMENT;
  const int64_t blk = fmt == FP4_FMT_MX ? 32 : 16;
  if (rows < 1 || k < blk || k % blk != 0) return FP4_INVALID_ARGUMENT;
  if (rows >= kMaxDim || k >= kMaxDim || ldx >= kMaxDim || ld_codes >= kMaxDim || ld_scales >= kMaxDim)
    return FP4_INVALID_ARGUMENT;
  const int64_t esize = x_dtype == FP4_DT_F32 ? 4 : 2;
  if (ldx < k || (ldx * esize) % 16 != 0 || !aligned(x, 16)) return FP4_INVALID_ARGUMENT;
  if (flags & FP4_LAYOUT_PANEL) {
    if (fmt != FP4_FMT_MX) return FP4_UNSUPPORTED;
    if (ld_codes != 0 || ld_scales != 0 || !aligned(codes, 16) || !aligned(scales, 4)) return FP4_INVALID_ARGUMENT;
  } else {
    if (ld_codes < k / 2 || ld_codes % 4 != 0 || !aligned(codes, 4)) return FP4_INVALID_ARGUMENT;
    if (ld_scales < k / blk) return FP4_INVALID_ARGUMENT;
  }
  if (fmt == FP4_FMT_MX) {
    if (tensor_scale) return FP4_INVALID_ARGUMENT;
    if (flags & ~(FP4_PRO_RMSNORM | FP4_PRO_GELU | FP4_LAYOUT_PANEL)) return FP4_INVALID_ARGUMENT;
    if ((flags & FP4_PRO_RMSNORM) && (flags & FP4_PRO_GELU)) return FP4_INVALID_ARGUMENT;
  } else {
    if (!tensor_scale || !aligned(tensor_scale, 4)) return FP4_INVALID_ARGUMENT;
    if (flags & (FP4_PRO_RMSNORM | FP4_PRO_GELU)) return FP4_UNSUPPORTED;
    if (flags & ~FP4_TENSOR_SCALE_GIVEN) return FP4_INVALID_ARGUMENT;
  }
  return FP4_OK;
}

fp4_status check_gemm(int fmt, const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as, const float* a_ts,
                      const uint8_t* b, int64_t ldb, const uint8_t* bs, int64_t ld_bs, const float* b_ts, int64_t m,
                      int64_t n, int64_t k, const void* c, int c_dtype, int64_t ldc, const float* residual) {
  if (fmt != FP4_FMT_MX && fmt != FP4_FMT_NV) return FP4_INVALID_ARGUMENT;
  if (!a || !as || !b || !bs || !c) return FP4_INVALID_ARGUMENT;
  const int64_t blk = fmt == FP4_FMT_MX ? 32 : 16;
  if (m < 1 || n < 1 || k < blk || k % blk != 0) return FP4_INVALID_ARGUMENT;
  // tile arithmetic is 32-bit; buffer offsets cover 256 rows of codes/scales
  if (m >= kMaxDim - 256 || n >= kMaxDim - 256 || k > ((int64_t)1 << 24)) return FP4_INVALID_ARGUMENT;
  if (lda < k / 2 || lda % 16 != 0 || !aligned(a, 16) || lda >= ((int64_t)1 << 23)) return FP4_INVALID_ARGUMENT;
  if (ldb < k / 2 || ldb % 16 != 0 || !aligned(b, 16) || ldb >= ((int64_t)1 << 23)) return FP4_INVALID_ARGUMENT;
  if (ld_as < k / blk || ld_bs < k / blk || ld_as >= ((int64_t)1 << 23) || ld_bs >= ((int64_t)1 << 23))
    return FP4_INVALID_ARGUMENT;
  if (c_dtype != FP4_DT_F32 && c_dtype != FP4_DT_BF16) return FP4_INVALID_ARGUMENT;
  if (ldc < n || ldc % 4 != 0 || ldc >= kMaxDim) return FP4_INVALID_ARGUMENT;
  if (!aligned(c, c_dtype == FP4_DT_F32 ? 16 : 8)) return FP4_INVALID_ARGUMENT;
  if (residual && (c_dtype != FP4_DT_F32 || !aligned(residual, 16))) return FP4_INVALID_ARGUMENT;
  if (fmt == FP4_FMT_MX) {
    if (a_ts || b_ts) return FP4_INVALID_ARGUMENT;
  } else {
    if (!a_ts || !b_ts || !aligned(a_ts, 4) || !aligned(b_ts, 4)) return FP4_INVALID_ARGUMENT;
  }
  const int64_t tiles = ((m + 255) / 256) * ((n + 255) / 256);
  if (tiles >= kMaxDim) return FP4_INVALID_ARGUMENT;
  return FP4_OK;
}

fp4_status check_output(int64_t m, int64_t n, const void* c, int c_dtype, int64_t ldc, const float* residual) {
  if (!c) return FP4_INVALID_ARGUMENT;
  if (c_dtype != FP4_DT_F32 && c_dtype != FP4_DT_BF16) return FP4_INVALID_ARGUMENT;
  if (ldc < n || ldc % 4 != 0 || ldc >= kMaxDim) return FP4_INVALID_ARGUMENT;
  if (!aligned(c, c_dtype == FP4_DT_F32 ? 16 : 8)) return FP4_INVALID_ARGUMENT;
  if (residual && (c_dtype != FP4_DT_F32 || !aligned(residual, 16))) return FP4_INVALID_ARGUMENT;
  const int64_t tiles = ((m + 255) / 256) * ((n + 255) / 256);
  if (tiles >= kMaxDim) return FP4_INVALID_ARGUMENT;
  return FP4_OK;
}

fp4_status check_gemm_panel(int fmt, const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                            int64_t m, int64_t n, int64_t k, const void* c, int c_dtype, int64_t ldc,
                            const float* residual) {
  if (fmt != FP4_FMT_MX && fmt != FP4_FMT_NV) return FP4_INVALID_ARGUMENT;
  if (!a || !as || !b || !bs) return FP4_INVALID_ARGUMENT;
  if (m < 1 || n < 1 || k < 32 || k % 32 != 0) return FP4_INVALID_ARGUMENT;
  // a panel's code bytes (k / 128 blocks of 16 KiB) stay below 2^31
  if (m >= kMaxDim - 256 || n >= kMaxDim - 256 || k > ((int64_t)1 << 23)) return FP4_INVALID_ARGUMENT;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(as, 4) || !aligned(bs, 4)) return FP4_INVALID_ARGUMENT;
  const fp4_status s = check_output(m, n, c, c_dtype, ldc, residual);
  if (s != FP4_OK) return s;
  if (fmt == FP4_FMT_NV) return FP4_UNSUPPORTED;
  return FP4_OK;
}

fp4_status check_quantize_lora(int fmt, const void* w, int w_dtype, int64_t rows, int64_t k, int64_t ldw,
                               const void* lora_b, int64_t ld_b, const void* lora_a, int64_t ld_a, int ab_dtype,
                               int64_t rank, float scale, const uint8_t* codes, int64_t ld_codes,
                               const uint8_t* scales, int64_t ld_scales, const float* tensor_scale, int flags) {
  if (fmt != FP4_FMT_MX && fmt != FP4_FMT_NV) return FP4_INVALID_ARGUMENT;
  if (!lora_b || !lora_a) return FP4_INVALID_ARGUMENT;
  if (ab_dtype != FP4_DT_F32 && ab_dtype != FP4_DT_BF16) return FP4_INVALID_ARGUMENT;
  if (rank < 1 || rank > 64) return FP4_INVALID_ARGUMENT;
  if (ld_b < rank || ld_a < k || ld_b >= kMaxDim || ld_a >= kMaxDim) return FP4_INVALID_ARGUMENT;
  const uintptr_t ab_size = ab_dtype == FP4_DT_F32 ? 4 : 2;
  if (!aligned(lora_b, ab_size) || !aligned(lora_a, ab_size)) return FP4_INVALID_ARGUMENT;
  if (!(scale - scale == 0.0f)) return FP4_INVALID_ARGUMENT;  // NaN or infinite
  // no prologues: MX takes only the panel layout flag, NV only a given tensor
  // scale (NV with the panel layout is refused by check_quantize)
  if (fmt == FP4_FMT_MX && (flags & ~FP4_LAYOUT_PANEL)) return FP4_INVALID_ARGUMENT;
  if (fmt == FP4_FMT_NV && (flags & ~(FP4_TENSOR_SCALE_GIVEN | FP4_LAYOUT_PANEL))) return FP4_INVALID_ARGUMENT;
  // the weight, the outputs and the tensor scale as for fp4_quantize
  return check_quantize(fmt, w, w_dtype, rows, k, ldw, codes, ld_codes, scales, ld_scales, tensor_scale, flags);
}

}  // namespace

extern "C" {

FP4_API fp4_status fp4_quantize(int fmt, const void* x, int x_dtype, int64_t rows, int64_t k, int64_t ldx,
                                uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                                float* tensor_scale, int flags, void* stream) {
  try {
    const fp4_status s =
        check_quantize(fmt, x, x_dtype, rows, k, ldx, codes, ld_codes, scales, ld_scales, tensor_scale, flags);
    if (s != FP4_OK) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int bf16 = x_dtype == FP4_DT_BF16;
    if (fmt == FP4_FMT_MX) {
      const int pro = (flags & FP4_PRO_RMSNORM) ? 1 : ((flags & FP4_PRO_GELU) ? 2 : 0);
      if (flags & FP4_LAYOUT_PANEL)
        return from_hip(fp4r::launch_quant_mx_panel(x, bf16, rows, k, ldx, codes, scales, pro, st));
      return from_hip(fp4r::launch_quant_mx(x, bf16, rows, k, ldx, codes, ld_codes, scales, ld_scales, pro, st));
    }
    return from_hip(fp4r::launch_quant_nv(x, bf16, rows, k, ldx, codes, ld_codes, scales, ld_scales, tensor_scale,
                                          (flags & FP4_TENSOR_SCALE_GIVEN) ? 1 : 0, st));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status fp4_gemm(int fmt, const uint8_t* a_codes, int64_t lda, const uint8_t* a_scales, int64_t ld_as,
                            const float* a_ts, const uint8_t* b_codes, int64_t ldb, const uint8_t* b_scales,
                            int64_t ld_bs, const float* b_ts, int64_t m, int64_t n, int64_t k, void* c, int c_dtype,
                            int64_t ldc, const float* residual, void* stream) {
  try {
    const fp4_status s = check_gemm(fmt, a_codes, lda, a_scales, ld_as, a_ts, b_codes, ldb, b_scales, ld_bs, b_ts, m,
                                    n, k, c, c_dtype, ldc, residual);
    if (s != FP4_OK) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int bf16 = c_dtype == FP4_DT_BF16;
    if (fmt == FP4_FMT_MX)
      return from_hip(fp4r::launch_gemm_mx(a_codes, lda, a_scales, ld_as, b_codes, ldb, b_scales, ld_bs, m, n, k, c,
                                           bf16, ldc, residual, st));
    return from_hip(fp4r::launch_gemm_nv(a_codes, lda, a_scales, ld_as, a_ts, b_codes, ldb, b_scales, ld_bs, b_ts, m,
                                         n, k, c, bf16, ldc, residual, st));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status fp4_panel_bytes(int64_t rows, int64_t k, int64_t* code_bytes, int64_t* scale_bytes) {
  if (!code_bytes || !scale_bytes || rows < 1 || k < 32 || k % 32 != 0) return FP4_INVALID_ARGUMENT;
  if (rows >= kMaxDim || k >= kMaxDim) return FP4_INVALID_ARGUMENT;
  const int64_t blocks = ((rows + 255) / 256) * ((k + 127) / 128);
  *code_bytes = blocks * 16384;
  *scale_bytes = blocks * 1024;
  return FP4_OK;
}

FP4_API fp4_status fp4_gemm_panel(int fmt, const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                                  const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, void* c, int c_dtype,
                                  int64_t ldc, const float* residual, void* stream) {
  try {
    const fp4_status s = check_gemm_panel(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, c, c_dtype, ldc, residual);
    if (s != FP4_OK) return s;
    return from_hip(fp4r::launch_gemm_mx_panel(a_codes, a_scales, b_codes, b_scales, m, n, k, c,
                                               c_dtype == FP4_DT_BF16, ldc, residual, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

namespace {
fp4_status gemm_panel_gelu(int fmt, const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                           const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, uint8_t* out_codes,
                           uint8_t* out_scales, int exact, void* stream) {
  if (fmt != FP4_FMT_MX && fmt != FP4_FMT_NV) return FP4_INVALID_ARGUMENT;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !out_codes || !out_scales) return FP4_INVALID_ARGUMENT;
  if (m < 1 || n < 1 || k < 32 || k % 32 != 0) return FP4_INVALID_ARGUMENT;
  if (m >= kMaxDim - 256 || n >= kMaxDim - 256 || k > ((int64_t)1 << 23)) return FP4_INVALID_ARGUMENT;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4) ||
      !aligned(out_codes, 16) || !aligned(out_scales, 4))
    return FP4_INVALID_ARGUMENT;
  const int64_t tiles = ((m + 255) / 256) * ((n + 255) / 256);
  if (tiles >= kMaxDim) return FP4_INVALID_ARGUMENT;
  if (fmt == FP4_FMT_NV || m % 256 != 0 || n % 256 != 0) return FP4_UNSUPPORTED;
  return from_hip(fp4r::launch_gemm_mx_panel_gelu(a_codes, a_scales, b_codes, b_scales, m, n, k, out_codes, out_scales,
                                                  exact, static_cast<hipStream_t>(stream)));
}
}  // namespace

FP4_API fp4_status fp4_gemm_panel_gelu(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t m, int64_t n,
                                       int64_t k, uint8_t* out_codes, uint8_t* out_scales, void* stream) {
  try {
    return gemm_panel_gelu(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, out_codes, out_scales, 0, stream);
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status fp4_gemm_panel_gelu_f32(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                           const uint8_t* b_codes, const uint8_t* b_scales, int64_t m, int64_t n,
                                           int64_t k, uint8_t* out_codes, uint8_t* out_scales, void* stream) {
  try {
    return gemm_panel_gelu(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, out_codes, out_scales, 1, stream);
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status fp4_gemm_panel_euler(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                        const uint8_t* b_codes, const uint8_t* b_scales, int64_t m, int64_t n,
                                        int64_t k, const float* residual, const float* x, float* x_out, int64_t ldx,
                                        float t_cur, float t_next, void* stream) {
  try {
    if (!residual || !x || !aligned(x, 16)) return FP4_INVALID_ARGUMENT;
    const fp4_status s =
        check_gemm_panel(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, x_out, FP4_DT_F32, ldx, residual);
    if (s != FP4_OK) return s;
    const float dt = t_next - t_cur;  // fp32 subtraction, as euler_step
    return from_hip(fp4r::launch_gemm_mx_panel_euler(a_codes, a_scales, b_codes, b_scales, m, n, k, residual, x,
                                                     x_out, ldx, dt, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status fp4_gemm_panel_euler_reward(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                               const uint8_t* b_codes, const uint8_t* b_scales, int64_t m, int64_t n,
                                               int64_t k, const float* residual, const float* x, float* x_out,
                                               int64_t ldx, float t_cur, float t_next, const float* u,
                                               int64_t rows_per_cand, float* partials, float* rewards, void* stream) {
  try {
    if (!residual || !x || !aligned(x, 16)) return FP4_INVALID_ARGUMENT;
    if (!u || !aligned(u, 16) || !partials || !aligned(partials, 4) || !rewards || !aligned(rewards, 4))
      return FP4_INVALID_ARGUMENT;
    if (rows_per_cand < 1 || rows_per_cand >= kMaxDim) return FP4_INVALID_ARGUMENT;
    const fp4_status s =
        check_gemm_panel(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, x_out, FP4_DT_F32, ldx, residual);
    if (s != FP4_OK) return s;
    if (m % rows_per_cand != 0) return FP4_INVALID_ARGUMENT;
    // the epilogue sums whole waves (128 x 128 values) of full 256 x 256 tiles
    if (m % 256 != 0 || n % 256 != 0 || rows_per_cand % 128 != 0) return FP4_UNSUPPORTED;
    const float dt = t_next - t_cur;  // fp32 subtraction, as euler_step
    return from_hip(fp4r::launch_gemm_mx_panel_euler_reward(a_codes, a_scales, b_codes, b_scales, m, n, k, residual,
                                                            x, x_out, ldx, dt, u, rows_per_cand, partials, rewards,
                                                            static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status fp4_gemm_panel_euler_reward_noalloc(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t m,
                                                       int64_t n, int64_t k, const float* residual, const float* x,
                                                       float* x_out, int64_t ldx, float t_cur, float t_next,
                                                       const float* u, int64_t rows_per_cand, float* rewards,
                                                       void* stream) {
  try {
    if (!residual || !x || !aligned(x, 16)) return FP4_INVALID_ARGUMENT;
    if (!u || !aligned(u, 16) || !rewards || !aligned(rewards, 4)) return FP4_INVALID_ARGUMENT;
    if (rows_per_cand < 1 || rows_per_cand >= kMaxDim) return FP4_INVALID_ARGUMENT;
    const fp4_status s =
        check_gemm_panel(fmt, a_codes, a_scales, b_codes, b_scales, m, n, k, x_out, FP4_DT_F32, ldx, residual);
    if (s != FP4_OK) return s;
    if (m % rows_per_cand != 0) return FP4_INVALID_ARGUMENT;
    if (m % 256 != 0 || n % 256 != 0 || rows_per_cand % 128 != 0) return FP4_UNSUPPORTED;
    // the library-owned partial sums: one float per wave tile
    if ((m / 256) * (n / 256) * 4 > fp4r::kNoAllocPartials) return FP4_INVALID_ARGUMENT;
    const float dt = t_next - t_cur;  // fp32 subtraction, as euler_step
    return from_hip(fp4r::launch_gemm_mx_panel_euler_reward_noalloc(a_codes, a_scales, b_codes, b_scales, m, n, k,
                                                                    residual, x, x_out, ldx, dt, u, rows_per_cand,
                                                                    rewards, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status euler_step(float* x_out, const float* x, const void* v, int v_dtype, int64_t numel, float t_cur,
                              float t_next, void* stream) {
  try {
    if (!x_out || !x || !v || numel < 1) return FP4_INVALID_ARGUMENT;
    if (v_dtype != FP4_DT_F32 && v_dtype != FP4_DT_BF16) return FP4_INVALID_ARGUMENT;
    if (!aligned(x_out, 16) || !aligned(x, 16) || !aligned(v, 16)) return FP4_INVALID_ARGUMENT;
    return from_hip(fp4r::launch_euler(x_out, x, v, v_dtype == FP4_DT_BF16, numel, t_cur, t_next,
                                       static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status fp4_proxy_reward(const float* x, int64_t n_cand, int64_t rows_per_cand, int64_t dim, int64_t ldx,
                                    const float* u, float* rewards, void* stream) {
  try {
    if (!x || !rewards || n_cand < 1 || rows_per_cand < 1 || dim < 4 || dim % 4 != 0) return FP4_INVALID_ARGUMENT;
    if (n_cand >= kMaxDim || rows_per_cand >= kMaxDim || ldx >= kMaxDim) return FP4_INVALID_ARGUMENT;
    if (ldx < dim || ldx % 4 != 0 || !aligned(x, 16) || !aligned(rewards, 4)) return FP4_INVALID_ARGUMENT;
    if (u && !aligned(u, 16)) return FP4_INVALID_ARGUMENT;
    return from_hip(
        fp4r::launch_proxy_reward(x, n_cand, rows_per_cand, dim, ldx, u, rewards, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status select_topk_bottomk(const float* rewards, int64_t n, int64_t k_top, int64_t k_bottom,
                                       int32_t* top_idx, int32_t* bottom_idx, float* r_norm, void* stream) {
  try {
    if (!rewards || n < 1 || n > 65536 || k_top < 0 || k_bottom < 0 || k_top + k_bottom > n)
      return FP4_INVALID_ARGUMENT;
    if ((k_top > 0 && !top_idx) || (k_bottom > 0 && !bottom_idx)) return FP4_INVALID_ARGUMENT;
    if (!aligned(rewards, 4) || (top_idx && !aligned(top_idx, 4)) || (bottom_idx && !aligned(bottom_idx, 4)) ||
        (r_norm && !aligned(r_norm, 4)))
      return FP4_INVALID_ARGUMENT;
    return from_hip(fp4r::launch_select(rewards, n, k_top, k_bottom, top_idx, bottom_idx, r_norm,
                                        static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API const char* fp4_status_str(fp4_status s) {
  switch (s) {
    case FP4_OK: return "ok";
    case FP4_INVALID_ARGUMENT: return "invalid argument";
    case FP4_UNSUPPORTED: return "unsupported";
    case FP4_DEVICE_ERROR: return "device error";
    case FP4_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

FP4_API fp4_status fp4_quantize_lora(int fmt, const void* w, int w_dtype, int64_t rows, int64_t k, int64_t ldw,
                                     const void* lora_b, int64_t ld_b, const void* lora_a, int64_t ld_a, int ab_dtype,
                                     int64_t rank, float scale, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                                     int64_t ld_scales, float* tensor_scale, int flags, void* stream) {
  try {
    const fp4_status s = check_quantize_lora(fmt, w, w_dtype, rows, k, ldw, lora_b, ld_b, lora_a, ld_a, ab_dtype, rank,
                                             scale, codes, ld_codes, scales, ld_scales, tensor_scale, flags);
    if (s != FP4_OK) return s;
    if (fmt == FP4_FMT_NV)
      return from_hip(fp4r::launch_quant_nv_lora(w, w_dtype == FP4_DT_BF16, rows, k, ldw, lora_b, ld_b, lora_a, ld_a,
                                                 ab_dtype == FP4_DT_BF16, (int)rank, scale, codes, ld_codes, scales,
                                                 ld_scales, tensor_scale, (flags & FP4_TENSOR_SCALE_GIVEN) ? 1 : 0,
                                                 static_cast<hipStream_t>(stream)));
    return from_hip(fp4r::launch_quant_mx_lora(w, w_dtype == FP4_DT_BF16, rows, k, ldw, lora_b, ld_b, lora_a, ld_a,
                                               ab_dtype == FP4_DT_BF16, (int)rank, scale, codes, ld_codes, scales,
                                               ld_scales, (flags & FP4_LAYOUT_PANEL) ? 1 : 0,
                                               static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status fp4_quantize_nv_grouped(const void* x, int x_dtype, int64_t rows, int64_t k, int64_t ldx,
                                           int64_t rows_per_group, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                                           int64_t ld_scales, float* tensor_scales, int flags, void* stream) {
  try {
    const fp4_status s = check_quantize(FP4_FMT_NV, x, x_dtype, rows, k, ldx, codes, ld_codes, scales, ld_scales,
                                        tensor_scales, flags);
    if (s != FP4_OK) return s;
    if (rows_per_group < 1 || rows % rows_per_group != 0) return FP4_INVALID_ARGUMENT;
    return from_hip(fp4r::launch_quant_nv_grouped(x, x_dtype == FP4_DT_BF16, rows, k, ldx, rows_per_group, codes,
                                                  ld_codes, scales, ld_scales, tensor_scales,
                                                  (flags & FP4_TENSOR_SCALE_GIVEN) ? 1 : 0,
                                                  static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status fp4_gemm_nv_grouped(const uint8_t* a_codes, int64_t lda, const uint8_t* a_scales, int64_t ld_as,
                                       const float* a_ts, int64_t a_rows_per_group, const uint8_t* b_codes,
                                       int64_t ldb, const uint8_t* b_scales, int64_t ld_bs, const float* b_ts,
                                       int64_t m, int64_t n, int64_t k, void* c, int c_dtype, int64_t ldc,
                                       const float* residual, void* stream) {
  try {
    const fp4_status s = check_gemm(FP4_FMT_NV, a_codes, lda, a_scales, ld_as, a_ts, b_codes, ldb, b_scales, ld_bs,
                                    b_ts, m, n, k, c, c_dtype, ldc, residual);
    if (s != FP4_OK) return s;
    if (a_rows_per_group < 1 || m % a_rows_per_group != 0) return FP4_INVALID_ARGUMENT;
    // the grouped scales ride in the f16-MFMA kernel, which loads scale rows as words
    if (ld_as % 4 != 0 || ld_bs % 4 != 0 || !aligned(a_scales, 4) || !aligned(b_scales, 4)) return FP4_UNSUPPORTED;
    return from_hip(fp4r::launch_gemm_nv_f16(a_codes, lda, a_scales, ld_as, a_ts, b_codes, ldb, b_scales, ld_bs, b_ts,
                                             m, n, k, c, c_dtype == FP4_DT_BF16, ldc, residual,
                                             static_cast<hipStream_t>(stream), a_rows_per_group));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status fp4_nft_noise(const float* x0, const float* eps, const float* t, int64_t n, int64_t d, float* x_t,
                                 void* stream) {
  try {
    if (!x0 || !eps || !t || !x_t) return FP4_INVALID_ARGUMENT;
    if (n < 1 || n > 65535 || d < 4 || d % 4 != 0 || d >= ((int64_t)1 << 40)) return FP4_INVALID_ARGUMENT;
    if (!aligned(x0, 16) || !aligned(eps, 16) || !aligned(x_t, 16) || !aligned(t, 4)) return FP4_INVALID_ARGUMENT;
    return from_hip(fp4r::launch_nft_noise(x0, eps, t, n, d, x_t, static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API fp4_status fp4_nft_loss(const float* v_old, const float* v_theta, const float* x0, const float* eps,
                                const float* r, float beta, int64_t n, int64_t d, float* partials, float* terms,
                                float* loss, void* stream) {
  try {
    if (!v_old || !v_theta || !x0 || !eps || !r || !partials || !terms || !loss) return FP4_INVALID_ARGUMENT;
    if (n < 1 || n > 65535 || d < 4 || d % 4 != 0 || d >= ((int64_t)1 << 40)) return FP4_INVALID_ARGUMENT;
    if (!aligned(v_old, 16) || !aligned(v_theta, 16) || !aligned(x0, 16) || !aligned(eps, 16)) return FP4_INVALID_ARGUMENT;
    if (!aligned(r, 4) || !aligned(partials, 4) || !aligned(terms, 4) || !aligned(loss, 4)) return FP4_INVALID_ARGUMENT;
    if (!(beta - beta == 0.0f)) return FP4_INVALID_ARGUMENT;  // NaN or infinite
    return from_hip(fp4r::launch_nft_loss(v_old, v_theta, x0, eps, r, beta, n, d, partials, terms, loss,
                                          static_cast<hipStream_t>(stream)));
  } catch (...) {
    return FP4_INTERNAL;
  }
}

FP4_API int fp4_abi_version(void) { return 110; }

}  // extern "C"
