// Host-side launch entry points of the fp4rollout kernels (no device code, so
// the C ABI layer can be built with the host compiler).
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fp4r {

// ---- launch entry points (host side, defined in the kernel sources) ----
// Each returns the hipError_t of its launch(es); arguments are already validated.
hipError_t launch_quant_mx(const void* x, int x_bf16, int64_t rows, int64_t k, int64_t ldx,
                           uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                           int prologue, hipStream_t st);
hipError_t launch_quant_mx_panel(const void* x, int x_bf16, int64_t rows, int64_t k, int64_t ldx, uint8_t* codes,
                                 uint8_t* scales, int prologue, hipStream_t st);
hipError_t launch_quant_mx_lora(const void* w, int w_bf16, int64_t rows, int64_t k, int64_t ldw, const void* lb,
                                int64_t ldb, const void* la, int64_t lda, int ab_bf16, int rank, float scale,
                                uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, int panel,
                                hipStream_t st);
hipError_t launch_quant_nv_lora(const void* w, int w_bf16, int64_t rows, int64_t k, int64_t ldw, const void* lb,
                                int64_t ldb, const void* la, int64_t lda, int ab_bf16, int rank, float scale,
                                uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales, float* ts,
                                int scale_given, hipStream_t st);
// The NVFP4-style tensor-scale word: zero it before an amax pass (integer
// atomicMax on the float bits), then turn the amax into s_g = fl(amax / 2688),
// 1 where that is 0.
hipError_t launch_nv_scale_reset(float* ts, hipStream_t st);
hipError_t launch_nv_scale_finalize(float* ts, hipStream_t st);
hipError_t launch_quant_nv(const void* x, int x_bf16, int64_t rows, int64_t k, int64_t ldx,
                           uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                           float* tensor_scale, int scale_given, hipStream_t st);
hipError_t launch_gemm_mx(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as,
                          const uint8_t* b, int64_t ldb, const uint8_t* bs, int64_t ld_bs,
                          int64_t m, int64_t n, int64_t k, void* c, int c_bf16, int64_t ldc,
                          const float* residual, hipStream_t st);
hipError_t launch_gemm_mx_panel(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                                int64_t m, int64_t n, int64_t k, void* c, int c_bf16, int64_t ldc,
                                const float* residual, hipStream_t st);
// exact: GELU of the fp32 sums (erfc per element) instead of their bf16 rounding (table)
hipError_t launch_gemm_mx_panel_gelu(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                                     int64_t m, int64_t n, int64_t k, uint8_t* out_codes, uint8_t* out_scales,
                                     int exact, hipStream_t st);
hipError_t launch_gemm_mx_panel_euler(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                                      int64_t m, int64_t n, int64_t k, const float* residual, const float* x,
                                      float* x_out, int64_t ldx, float dt, hipStream_t st);
hipError_t launch_gemm_mx_panel_euler_reward(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                                             int64_t m, int64_t n, int64_t k, const float* residual, const float* x,
                                             float* x_out, int64_t ldx, float dt, const float* u, int64_t rows_per_cand,
                                             float* partials, float* rewards, hipStream_t st);
// The no-allocation variant of launch_gemm_mx_panel_euler_reward: the partial
// sums live in a library-owned device array of kNoAllocPartials floats per GPU.
constexpr int64_t kNoAllocPartials = (int64_t)1 << 18;
constexpr int kMaxDevices = 64;
hipError_t launch_gemm_mx_panel_euler_reward_noalloc(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                                                     const uint8_t* bs, int64_t m, int64_t n, int64_t k,
                                                     const float* residual, const float* x, float* x_out, int64_t ldx,
                                                     float dt, const float* u, int64_t rows_per_cand, float* rewards,
                                                     hipStream_t st);
hipError_t launch_gemm_nv(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as, const float* a_ts,
                          const uint8_t* b, int64_t ldb, const uint8_t* bs, int64_t ld_bs, const float* b_ts,
                          int64_t m, int64_t n, int64_t k, void* c, int c_bf16, int64_t ldc,
                          const float* residual, hipStream_t st);
hipError_t launch_gemm_nv_f16(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as, const float* a_ts,
                              const uint8_t* b, int64_t ldb, const uint8_t* bs, int64_t ld_bs, const float* b_ts,
                              int64_t m, int64_t n, int64_t k, void* c, int c_bf16, int64_t ldc, const float* residual,
                              hipStream_t st, int64_t a_rows_per_group = 0);
hipError_t launch_quant_nv_grouped(const void* x, int x_bf16, int64_t rows, int64_t k, int64_t ldx, int64_t rpg,
                                   uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                                   float* tensor_scales, int scale_given, hipStream_t st);
hipError_t launch_euler(float* x_out, const float* x, const void* v, int v_bf16, int64_t numel,
                        float t_cur, float t_next, hipStream_t st);
hipError_t launch_proxy_reward(const float* x, int64_t n_cand, int64_t rows_per_cand, int64_t dim,
                               int64_t ldx, const float* u, float* rewards, hipStream_t st);
hipError_t launch_nft_noise(const float* x0, const float* eps, const float* t, int64_t n, int64_t d, float* xt,
                            hipStream_t st);
hipError_t launch_nft_loss(const float* v_old, const float* v_theta, const float* x0, const float* eps,
                           const float* r, float beta, int64_t n, int64_t d, float* partials, float* terms,
                           float* loss, hipStream_t st);
hipError_t launch_select(const float* r, int64_t n, int64_t k_top, int64_t k_bottom,
                         int32_t* top, int32_t* bottom, float* r_norm, hipStream_t st);

}  // namespace fp4r
