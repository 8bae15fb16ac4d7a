"""MI355X-native FP4 exploration hot path (quantize, FP4 GEMM, Euler step,
proxy reward, seed selection) behind the C ABI in include/fp4rollout.h.

The binding loads libfp4rollout.so on first use and raises when it has not
been built; `inputs` holds the seeded synthetic workloads and needs no GPU.
"""
import importlib

_BINDING_NAMES = {
    "load_library", "Fp4Error", "QTensor", "quantize", "gemm", "euler", "proxy_reward", "select",
    "fp4_quantize", "fp4_gemm", "euler_step", "fp4_proxy_reward", "select_topk_bottomk", "fp4_abi_version",
    "status_str", "EXPORTS", "LIB_PATH", "FMT_MX", "FMT_NV", "DT_F32", "DT_BF16", "PRO_RMSNORM", "PRO_GELU",
    "TENSOR_SCALE_GIVEN", "LAYOUT_PANEL", "fp4_panel_bytes", "fp4_gemm_panel", "panel_bytes",
    "fp4_gemm_panel_euler", "gemm_euler", "fp4_gemm_panel_gelu", "gemm_gelu", "fp4_quantize_lora", "quantize_lora",
    "fp4_gemm_panel_euler_reward", "gemm_euler_reward", "fp4_quantize_nv_grouped", "quantize_nv_grouped",
    "fp4_gemm_nv_grouped", "fp4_nft_noise", "fp4_nft_loss", "nft_noise", "nft_loss",
    "fp4_gemm_panel_euler_reward_noalloc", "gemm_euler_reward_noalloc", "fp4_gemm_panel_gelu_f32",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        return getattr(importlib.import_module(".binding", __name__), name)
    if name in ("inputs", "rollout", "build"):
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
