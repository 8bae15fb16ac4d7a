// Host-only stand-ins for the kernel launchers (csrc/common_host.h), for the
// sanitizer build of the C-ABI layer: each records its name and returns
// hipSuccess without touching memory, so valid calls run the ABI's whole
// validation and dispatch on the CPU. fp4_stub_last_launch() names the
// launcher the last call reached.
#include "common_host.h"

namespace {
const char* g_last = "";
hipError_t hit(const char* name) {
  g_last = name;
  return hipSuccess;
}
}  // namespace

extern "C" __attribute__((visibility("default"))) const char* fp4_stub_last_launch() { return g_last; }
extern "C" __attribute__((visibility("default"))) void fp4_stub_reset() { g_last = ""; }

namespace fp4r {
hipError_t launch_quant_mx(const void*, int, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint8_t*, int64_t, int,
                           hipStream_t) { return hit("launch_quant_mx"); }
hipError_t launch_quant_mx_panel(const void*, int, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, int, hipStream_t) {
  return hit("launch_quant_mx_panel");
}
hipError_t launch_quant_mx_lora(const void*, int, int64_t, int64_t, int64_t, const void*, int64_t, const void*,
                                int64_t, int, int, float, uint8_t*, int64_t, uint8_t*, int64_t, int, hipStream_t) {
  return hit("launch_quant_mx_lora");
}
hipError_t launch_quant_nv_lora(const void*, int, int64_t, int64_t, int64_t, const void*, int64_t, const void*,
                                int64_t, int, int, float, uint8_t*, int64_t, uint8_t*, int64_t, float*, int,
                                hipStream_t) { return hit("launch_quant_nv_lora"); }
hipError_t launch_nv_scale_reset(float*, hipStream_t) { return hit("launch_nv_scale_reset"); }
hipError_t launch_nv_scale_finalize(float*, hipStream_t) { return hit("launch_nv_scale_finalize"); }
hipError_t launch_quant_nv(const void*, int, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint8_t*, int64_t, float*,
                           int, hipStream_t) { return hit("launch_quant_nv"); }
hipError_t launch_gemm_mx(const uint8_t*, int64_t, const uint8_t*, int64_t, const uint8_t*, int64_t, const uint8_t*,
                          int64_t, int64_t, int64_t, int64_t, void*, int, int64_t, const float*, hipStream_t) {
  return hit("launch_gemm_mx");
}
hipError_t launch_gemm_mx_panel(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t, int64_t,
                                int64_t, void*, int, int64_t, const float*, hipStream_t) {
  return hit("launch_gemm_mx_panel");
}
hipError_t launch_gemm_mx_panel_gelu(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t, int64_t,
                                     int64_t, uint8_t*, uint8_t*, int exact, hipStream_t) {
  return hit(exact ? "launch_gemm_mx_panel_gelu(exact)" : "launch_gemm_mx_panel_gelu");
}
hipError_t launch_gemm_mx_panel_euler(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t,
                                      int64_t, int64_t, const float*, const float*, float*, int64_t, float,
                                      hipStream_t) { return hit("launch_gemm_mx_panel_euler"); }
hipError_t launch_gemm_mx_panel_euler_reward(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t,
                                             int64_t, int64_t, const float*, const float*, float*, int64_t, float,
                                             const float*, int64_t, float*, float*, hipStream_t) {
  return hit("launch_gemm_mx_panel_euler_reward");
}
hipError_t launch_gemm_mx_panel_euler_reward_noalloc(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*,
                                                     int64_t, int64_t, int64_t, const float*, const float*, float*,
                                                     int64_t, float, const float*, int64_t, float*, hipStream_t) {
  return hit("launch_gemm_mx_panel_euler_reward_noalloc");
}
hipError_t launch_gemm_nv(const uint8_t*, int64_t, const uint8_t*, int64_t, const float*, const uint8_t*, int64_t,
                          const uint8_t*, int64_t, const float*, int64_t, int64_t, int64_t, void*, int, int64_t,
                          const float*, hipStream_t) { return hit("launch_gemm_nv"); }
hipError_t launch_gemm_nv_f16(const uint8_t*, int64_t, const uint8_t*, int64_t, const float*, const uint8_t*, int64_t,
                              const uint8_t*, int64_t, const float*, int64_t, int64_t, int64_t, void*, int, int64_t,
                              const float*, hipStream_t, int64_t) { return hit("launch_gemm_nv_f16"); }
hipError_t launch_quant_nv_grouped(const void*, int, int64_t, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint8_t*,
                                   int64_t, float*, int, hipStream_t) { return hit("launch_quant_nv_grouped"); }
hipError_t launch_euler(float*, const float*, const void*, int, int64_t, float, float, hipStream_t) {
  return hit("launch_euler");
}
hipError_t launch_proxy_reward(const float*, int64_t, int64_t, int64_t, int64_t, const float*, float*, hipStream_t) {
  return hit("launch_proxy_reward");
}
hipError_t launch_nft_noise(const float*, const float*, const float*, int64_t, int64_t, float*, hipStream_t) {
  return hit("launch_nft_noise");
}
hipError_t launch_nft_loss(const float*, const float*, const float*, const float*, const float*, float, int64_t,
                           int64_t, float*, float*, float*, hipStream_t) { return hit("launch_nft_loss"); }
hipError_t launch_select(const float*, int64_t, int64_t, int64_t, int32_t*, int32_t*, float*, hipStream_t) {
  return hit("launch_select");
}
}  // namespace fp4r
