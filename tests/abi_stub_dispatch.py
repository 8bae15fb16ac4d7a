"""Valid calls through the C ABI reach the right kernel launcher. Run only
against the sanitizer build of the ABI layer, whose launchers are recording
stubs (tests/abi_stubs.cpp): the pointers below are never dereferenced.
Collected only when named explicitly (test_abi_sanitized.py does)."""
import ctypes
import os

import pytest

import fp4_quantized_diffusion_amd as fq

P, P2, P3 = 0x10000, 0x20000, 0x30000
STREAM = None


@pytest.fixture(scope="module")
def lib():
    path = os.environ.get("FP4_ABI_TEST_LIB")
    if not path:
        pytest.fail("run through test_abi_sanitized.py")
    lib = fq.load_library(path)
    stub = ctypes.CDLL(path)
    stub.fp4_stub_last_launch.restype = ctypes.c_char_p
    return stub


def last(stub):
    return stub.fp4_stub_last_launch().decode()


CASES = [
    ("fp4_quantize", (0, P, 0, 4, 64, 64, P2, 32, P3, 2, None, 0, STREAM), "launch_quant_mx"),
    ("fp4_quantize", (0, P, 1, 4, 64, 64, P2, 32, P3, 2, None, 1, STREAM), "launch_quant_mx"),
    ("fp4_quantize", (0, P, 0, 4, 64, 64, P2, 0, P3, 0, None, 0x202, STREAM), "launch_quant_mx_panel"),
    ("fp4_quantize", (1, P, 0, 4, 64, 64, P2, 32, P3, 4, P, 0, STREAM), "launch_quant_nv"),
    ("fp4_quantize", (1, P, 0, 4, 64, 64, P2, 32, P3, 4, P, 0x100, STREAM), "launch_quant_nv"),
    ("fp4_gemm", (0, P, 32, P3, 2, None, P2, 32, P3, 2, None, 8, 8, 64, P, 0, 8, None, STREAM), "launch_gemm_mx"),
    ("fp4_gemm", (1, P, 32, P3, 4, P, P2, 32, P3, 4, P2, 8, 8, 64, P, 1, 8, None, STREAM), "launch_gemm_nv"),
    ("fp4_gemm_panel", (0, P, P3, P2, P3, 8, 8, 64, P, 0, 8, P2, STREAM), "launch_gemm_mx_panel"),
    ("fp4_gemm_panel_gelu", (0, P, P3, P2, P3, 256, 512, 64, P, P3, STREAM), "launch_gemm_mx_panel_gelu"),
    ("fp4_gemm_panel_gelu_f32", (0, P, P3, P2, P3, 256, 512, 64, P, P3, STREAM), "launch_gemm_mx_panel_gelu(exact)"),
    ("fp4_gemm_panel_euler", (0, P, P3, P2, P3, 8, 8, 64, P2, P3, P, 8, 1.0, 0.5, STREAM),
     "launch_gemm_mx_panel_euler"),
    ("fp4_gemm_panel_euler_reward", (0, P, P3, P2, P3, 256, 256, 64, P2, P3, P, 256, 1.0, 0.5, P2, 128, P3, P,
                                     STREAM), "launch_gemm_mx_panel_euler_reward"),
    ("fp4_gemm_panel_euler_reward_noalloc", (0, P, P3, P2, P3, 256, 256, 64, P2, P3, P, 256, 1.0, 0.5, P2, 128, P,
                                             STREAM), "launch_gemm_mx_panel_euler_reward_noalloc"),
    ("fp4_gemm_panel_euler_reward_noalloc", (0, P, P3, P2, P3, 256 * 512, 256 * 128, 64, P2, P3, P, 256 * 128, 1.0,
                                             0.5, P2, 128, P, STREAM), "launch_gemm_mx_panel_euler_reward_noalloc"),
    ("euler_step", (P, P2, P3, 0, 100, 1.0, 0.5, STREAM), "launch_euler"),
    ("fp4_proxy_reward", (P, 2, 3, 8, 8, None, P2, STREAM), "launch_proxy_reward"),
    ("select_topk_bottomk", (P, 8, 2, 2, P2, P3, None, STREAM), "launch_select"),
    ("fp4_quantize_lora", (0, P, 0, 4, 64, 64, P2, 8, P3, 64, 0, 8, 0.25, P2, 32, P3, 2, None, 0, STREAM),
     "launch_quant_mx_lora"),
    ("fp4_quantize_lora", (1, P, 0, 4, 64, 64, P2, 8, P3, 64, 0, 8, 0.25, P2, 32, P3, 4, P, 0, STREAM),
     "launch_quant_nv_lora"),
    ("fp4_quantize_nv_grouped", (P, 0, 8, 64, 64, 4, P2, 32, P3, 4, P, 0, STREAM), "launch_quant_nv_grouped"),
    ("fp4_gemm_nv_grouped", (P, 32, P3, 4, P, 4, P2, 32, P3, 4, P2, 8, 8, 64, P, 0, 8, None, STREAM),
     "launch_gemm_nv_f16"),
    ("fp4_nft_noise", (P, P, P2, 2, 8, P3, STREAM), "launch_nft_noise"),
    ("fp4_nft_loss", (P, P, P2, P3, P, 0.5, 2, 8, P2, P3, P, STREAM), "launch_nft_loss"),
]


@pytest.mark.parametrize("name,args,launcher", CASES, ids=[f"{c[0]}-{c[2]}-{i}" for i, c in enumerate(CASES)])
def test_valid_call_reaches_its_launcher(lib, name, args, launcher):
    lib.fp4_stub_reset()
    assert getattr(fq, name)(*args) == fq.binding.OK
    assert last(lib) == launcher


def test_rejected_call_reaches_no_launcher(lib):
    lib.fp4_stub_reset()
    assert fq.fp4_gemm(0, P, 32, P3, 2, None, P2, 32, P3, 2, None, 0, 8, 64, P, 0, 8, None, STREAM) != 0
    assert last(lib) == ""
