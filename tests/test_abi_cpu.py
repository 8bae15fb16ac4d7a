"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, and validates arguments on the host (returning a status before any
device work). No compute call reaches a device here: every call below is
rejected by validation, and the pointers are never dereferenced."""
import os
import re

import pytest

import fp4_quantized_diffusion_amd as fq
from fp4_quantized_diffusion_amd import build as fbuild

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fp4rollout.h")
P = 0x10000       # a fake, 64 KiB-aligned "device address" (never dereferenced)
P2 = 0x20000
P3 = 0x30000


@pytest.fixture(scope="module")
def lib():
    alt = os.environ.get("FP4_ABI_TEST_LIB")  # the sanitizer build of the ABI layer (test_abi_sanitized.py)
    if alt:
        return fq.load_library(alt)
    if not os.path.exists(fq.LIB_PATH):
        fbuild.build()
    return fq.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"FP4_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert set(names) == set(fq.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert fq.fp4_abi_version() == 110


def test_status_strings(lib):
    assert fq.status_str(0) == "ok"
    assert fq.status_str(1) == "invalid argument"
    assert fq.status_str(2) == "unsupported"
    assert fq.status_str(99) == "unknown status"


def q(**kw):
    a = dict(fmt=0, x=P, x_dtype=0, rows=4, k=64, ldx=64, codes=P2, ld_codes=32, scales=P3, ld_scales=2,
             tensor_scale=None, flags=0, stream=None)
    a.update(kw)
    return fq.fp4_quantize(*a.values())


@pytest.mark.parametrize("kw", [
    dict(fmt=2), dict(x=None), dict(codes=None), dict(scales=None), dict(x_dtype=5),
    dict(rows=0), dict(k=48), dict(k=0), dict(ldx=32), dict(ldx=66), dict(x=P + 4),
    dict(ld_codes=16), dict(ld_codes=34), dict(codes=P2 + 2), dict(ld_scales=1),
    dict(tensor_scale=P3), dict(flags=3), dict(flags=0x100), dict(flags=0x40),
    dict(fmt=1, tensor_scale=None), dict(fmt=1, k=24, ldx=64, tensor_scale=P3),
    dict(fmt=1, tensor_scale=P3 + 1), dict(rows=1 << 31),
])
def test_quantize_rejects(lib, kw):
    assert q(**kw) == fq.binding.INVALID_ARGUMENT


def test_quantize_nv_prologue_unsupported(lib):
    assert q(fmt=1, tensor_scale=P3, flags=1, ld_scales=4) == fq.binding.UNSUPPORTED


def g(**kw):
    a = dict(fmt=0, a=P, lda=32, a_s=P3, ld_as=2, a_ts=None, b=P2, ldb=32, b_s=P3, ld_bs=2, b_ts=None,
             m=8, n=8, k=64, c=P, c_dtype=0, ldc=8, residual=None, stream=None)
    a.update(kw)
    return fq.fp4_gemm(*a.values())


@pytest.mark.parametrize("kw", [
    dict(fmt=3), dict(a=None), dict(b=None), dict(a_s=None), dict(c=None), dict(m=0), dict(n=0),
    dict(k=48), dict(lda=16), dict(lda=40), dict(a=P + 8), dict(ldb=24), dict(ld_as=1), dict(ld_bs=1),
    dict(c_dtype=7), dict(ldc=6), dict(ldc=10), dict(c=P + 4), dict(c_dtype=1, c=P + 2),
    dict(c_dtype=1, residual=P2), dict(residual=P2 + 4), dict(a_ts=P3), dict(fmt=1),
    dict(fmt=1, a_ts=P3, b_ts=None), dict(k=1 << 25, lda=1 << 24, ldb=1 << 24, ld_as=1 << 20, ld_bs=1 << 20),
])
def test_gemm_rejects(lib, kw):
    assert g(**kw) == fq.binding.INVALID_ARGUMENT


@pytest.mark.parametrize("args", [
    (None, P, P2, 0, 16, 1.0, 0.5, None), (P, P, P2, 0, 0, 1.0, 0.5, None), (P, P, P2, 9, 16, 1.0, 0.5, None),
    (P + 4, P, P2, 0, 16, 1.0, 0.5, None), (P, P, P2 + 8, 1, 16, 1.0, 0.5, None),
])
def test_euler_rejects(lib, args):
    assert fq.euler_step(*args) == fq.binding.INVALID_ARGUMENT


@pytest.mark.parametrize("args", [
    (None, 2, 2, 8, 8, None, P2, None), (P, 0, 2, 8, 8, None, P2, None), (P, 2, 2, 6, 8, None, P2, None),
    (P, 2, 2, 8, 4, None, P2, None), (P, 2, 2, 8, 8, P3 + 4, P2, None), (P, 2, 2, 8, 8, None, None, None),
])
def test_reward_rejects(lib, args):
    assert fq.fp4_proxy_reward(*args) == fq.binding.INVALID_ARGUMENT


@pytest.mark.parametrize("args", [
    (None, 8, 2, 2, P, P2, None, None), (P, 0, 0, 0, P, P2, None, None), (P, 8, 5, 4, P, P2, None, None),
    (P, 8, -1, 2, P, P2, None, None), (P, 8, 2, 2, None, P2, None, None), (P, 8, 2, 2, P, None, None, None),
    (P, 65537, 2, 2, P, P2, None, None), (P + 2, 8, 2, 2, P, P2, None, None),
])
def test_select_rejects(lib, args):
    assert fq.select_topk_bottomk(*args) == fq.binding.INVALID_ARGUMENT


def test_panel_bytes(lib):
    import ctypes
    cb, sb = ctypes.c_int64(-1), ctypes.c_int64(-1)
    for rows, k, blocks in [(1, 32, 1), (256, 128, 1), (257, 128, 2), (300, 160, 4), (393216, 3072, 1536 * 24)]:
        assert fq.fp4_panel_bytes(rows, k, ctypes.addressof(cb), ctypes.addressof(sb)) == fq.binding.OK
        assert (cb.value, sb.value) == (blocks * 16384, blocks * 1024)
    assert fq.binding.panel_bytes(513, 4160) == (3 * 33 * 16384, 3 * 33 * 1024)
    for rows, k in [(0, 32), (4, 48), (4, 0), (1 << 31, 32)]:
        assert fq.fp4_panel_bytes(rows, k, ctypes.addressof(cb), ctypes.addressof(sb)) == fq.binding.INVALID_ARGUMENT
    assert fq.fp4_panel_bytes(4, 32, None, ctypes.addressof(sb)) == fq.binding.INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [
    dict(flags=0x200), dict(flags=0x200, ld_codes=0), dict(flags=0x200, ld_scales=0),
    dict(flags=0x200, ld_codes=0, ld_scales=0, codes=P2 + 4), dict(flags=0x200, ld_codes=0, ld_scales=0, scales=P3 + 2),
    dict(flags=0x203, ld_codes=0, ld_scales=0), dict(flags=0x400, ld_codes=0, ld_scales=0),
])
def test_quantize_panel_rejects(lib, kw):
    assert q(**kw) == fq.binding.INVALID_ARGUMENT


def test_quantize_panel_nv_unsupported(lib):
    assert q(fmt=1, tensor_scale=P3, flags=0x200, ld_codes=0, ld_scales=0) == fq.binding.UNSUPPORTED


def gp(**kw):
    a = dict(fmt=0, a=P, a_s=P3, b=P2, b_s=P3, m=8, n=8, k=64, c=P, c_dtype=0, ldc=8, residual=None, stream=None)
    a.update(kw)
    return fq.fp4_gemm_panel(*a.values())


@pytest.mark.parametrize("kw", [
    dict(fmt=3), dict(a=None), dict(b=None), dict(a_s=None), dict(b_s=None), dict(c=None), dict(m=0), dict(n=0),
    dict(k=0), dict(k=48), dict(k=(1 << 23) + 32), dict(a=P + 8), dict(b=P2 + 4), dict(a_s=P3 + 2), dict(b_s=P3 + 1),
    dict(c_dtype=7), dict(ldc=6), dict(ldc=10), dict(c=P + 4), dict(c_dtype=1, c=P + 2),
    dict(c_dtype=1, residual=P2), dict(residual=P2 + 4), dict(m=1 << 31),
])
def test_gemm_panel_rejects(lib, kw):
    assert gp(**kw) == fq.binding.INVALID_ARGUMENT


def test_gemm_panel_nv_unsupported(lib):
    assert gp(fmt=1) == fq.binding.UNSUPPORTED


def ge(**kw):
    a = dict(fmt=0, a=P, a_s=P3, b=P2, b_s=P3, m=8, n=8, k=64, residual=P2, x=P3, x_out=P, ldx=8,
             t_cur=1.0, t_next=5.0 / 6.0, stream=None)
    a.update(kw)
    return fq.fp4_gemm_panel_euler(*a.values())


@pytest.mark.parametrize("kw", [
    dict(fmt=3), dict(a=None), dict(b_s=None), dict(residual=None), dict(x=None), dict(x_out=None),
    dict(x=P3 + 4), dict(residual=P2 + 8), dict(x_out=P + 4), dict(m=0), dict(k=48), dict(ldx=6), dict(ldx=10),
    dict(a=P + 8), dict(a_s=P3 + 2),
])
def test_gemm_panel_euler_rejects(lib, kw):
    assert ge(**kw) == fq.binding.INVALID_ARGUMENT


def test_gemm_panel_euler_nv_unsupported(lib):
    assert ge(fmt=1) == fq.binding.UNSUPPORTED


def gg(**kw):
    a = dict(fmt=0, a=P, a_s=P3, b=P2, b_s=P3, m=256, n=256, k=64, oc=P, os=P3, stream=None)
    a.update(kw)
    return fq.fp4_gemm_panel_gelu(*a.values())


@pytest.mark.parametrize("kw", [
    dict(fmt=3), dict(a=None), dict(b_s=None), dict(oc=None), dict(os=None), dict(m=0), dict(k=48),
    dict(oc=P + 8), dict(os=P3 + 2), dict(a=P + 8), dict(a_s=P3 + 2),
])
def test_gemm_panel_gelu_rejects(lib, kw):
    assert gg(**kw) == fq.binding.INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(fmt=1), dict(m=300), dict(n=128)])
def test_gemm_panel_gelu_unsupported(lib, kw):
    assert gg(**kw) == fq.binding.UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(fmt=3), dict(a=None), dict(oc=None), dict(m=0), dict(k=48), dict(oc=P + 8)])
def test_gemm_panel_gelu_f32_rejects(lib, kw):
    a = dict(fmt=0, a=P, a_s=P3, b=P2, b_s=P3, m=256, n=256, k=64, oc=P, os=P3, stream=None)
    a.update(kw)
    assert fq.fp4_gemm_panel_gelu_f32(*a.values()) == fq.binding.INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(fmt=1), dict(m=300), dict(n=128)])
def test_gemm_panel_gelu_f32_unsupported(lib, kw):
    a = dict(fmt=0, a=P, a_s=P3, b=P2, b_s=P3, m=256, n=256, k=64, oc=P, os=P3, stream=None)
    a.update(kw)
    assert fq.fp4_gemm_panel_gelu_f32(*a.values()) == fq.binding.UNSUPPORTED


def ql(**kw):
    a = dict(fmt=0, w=P, w_dtype=0, rows=4, k=64, ldw=64, b=P2, ld_b=8, a=P3, ld_a=64, ab_dtype=0, rank=8, scale=0.25,
             codes=P2, ld_codes=32, scales=P3, ld_scales=2, ts=None, flags=0, stream=None)
    a.update(kw)
    return fq.fp4_quantize_lora(*a.values())


@pytest.mark.parametrize("kw", [
    dict(fmt=2), dict(w=None), dict(b=None), dict(a=None), dict(codes=None), dict(scales=None), dict(w_dtype=5),
    dict(ab_dtype=3), dict(rank=0), dict(rank=65), dict(ld_b=7), dict(ld_a=32), dict(rows=0), dict(k=48),
    dict(ldw=32), dict(w=P + 4), dict(b=P2 + 2), dict(ab_dtype=1, a=P3 + 1), dict(scale=float("nan")),
    dict(scale=float("inf")), dict(flags=0x1), dict(flags=0x2), dict(flags=0x100), dict(ld_codes=16),
    dict(flags=0x200), dict(rows=1 << 31), dict(ts=P),
])
def test_quantize_lora_rejects(lib, kw):
    assert ql(**kw) == fq.binding.INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [
    dict(ts=None), dict(ts=P + 2), dict(flags=0x1), dict(flags=0x2), dict(k=40, ldw=40, ld_a=40),
    dict(ld_scales=3), dict(ld_codes=30),
])
def test_quantize_lora_nv_rejects(lib, kw):
    """NVFP4-style: a tensor-scale word is required (4-byte aligned), blocks of
    16 along k, no prologue, scale rows of at least k / 16 bytes."""
    a = dict(fmt=1, ld_scales=4, ts=P)
    a.update(kw)
    assert ql(**a) == fq.binding.INVALID_ARGUMENT


def test_quantize_lora_nv_panel_unsupported(lib):
    assert ql(fmt=1, ts=P, ld_codes=0, ld_scales=0, flags=0x200) == fq.binding.UNSUPPORTED


def test_rollout_lora_entries_per_block():
    """Host-side check of the rollout's adapter list (no device work)."""
    import torch
    from fp4_quantized_diffusion_amd.rollout import Fp4Rollout
    w = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        Fp4Rollout([w] * 4, [w] * 4, torch.zeros(4), lora=([None] * 3, [None] * 4))
    ro = Fp4Rollout([w] * 4, [w] * 4, torch.zeros(4))
    assert ro.lora1 == [None] * 4 and ro.lora2 == [None] * 4


def ger(**kw):
    a = dict(fmt=0, a=P, a_s=P3, b=P2, b_s=P3, m=256, n=256, k=64, residual=P2, x=P3, x_out=P, ldx=256,
             t_cur=1.0, t_next=5.0 / 6.0, u=P2, rows_per_cand=128, partials=P3, rewards=P, stream=None)
    a.update(kw)
    return fq.fp4_gemm_panel_euler_reward(*a.values())


@pytest.mark.parametrize("kw", [
    dict(fmt=3), dict(a=None), dict(residual=None), dict(x=None), dict(x_out=None), dict(u=None), dict(u=P2 + 4),
    dict(partials=None), dict(partials=P3 + 2), dict(rewards=None), dict(rewards=P + 1), dict(rows_per_cand=0),
    dict(rows_per_cand=96), dict(m=0), dict(k=48), dict(ldx=250), dict(x=P3 + 4),
])
def test_gemm_panel_euler_reward_rejects(lib, kw):
    assert ger(**kw) == fq.binding.INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(fmt=1), dict(m=384, rows_per_cand=128), dict(n=128, ldx=128),
                                dict(rows_per_cand=64)])
def test_gemm_panel_euler_reward_unsupported(lib, kw):
    assert ger(**kw) == fq.binding.UNSUPPORTED


def qg(**kw):
    a = dict(x=P, x_dtype=0, rows=8, k=64, ldx=64, rpg=4, codes=P2, ld_codes=32, scales=P3, ld_scales=4, ts=P,
             flags=0, stream=None)
    a.update(kw)
    return fq.fp4_quantize_nv_grouped(*a.values())


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(ts=None), dict(ts=P + 2), dict(rpg=0), dict(rpg=3), dict(rpg=16), dict(k=24),
    dict(flags=0x400), dict(ld_scales=3), dict(x_dtype=4),
])
def test_quantize_nv_grouped_rejects(lib, kw):
    assert qg(**kw) == fq.binding.INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(flags=0x200), dict(flags=0x1)])
def test_quantize_nv_grouped_unsupported(lib, kw):
    """The panel layout and the prologues are MX-only, as for fp4_quantize."""
    assert qg(**kw) == fq.binding.UNSUPPORTED


def gng(**kw):
    a = dict(a=P, lda=32, a_s=P3, ld_as=4, a_ts=P, rpg=4, b=P2, ldb=32, b_s=P3, ld_bs=4, b_ts=P2, m=8, n=8, k=64,
             c=P, c_dtype=0, ldc=8, residual=None, stream=None)
    a.update(kw)
    return fq.fp4_gemm_nv_grouped(*a.values())


@pytest.mark.parametrize("kw", [
    dict(a=None), dict(a_ts=None), dict(b_ts=None), dict(rpg=0), dict(rpg=3), dict(m=0), dict(k=8), dict(ldc=6),
])
def test_gemm_nv_grouped_rejects(lib, kw):
    assert gng(**kw) == fq.binding.INVALID_ARGUMENT


def test_gemm_nv_grouped_unaligned_scale_rows_unsupported(lib):
    assert gng(ld_as=5) == fq.binding.UNSUPPORTED


@pytest.mark.parametrize("args", [
    (None, P, P2, 2, 8, P3, None), (P, P, P2, 0, 8, P3, None), (P, P, P2, 70000, 8, P3, None),
    (P, P, P2, 2, 6, P3, None), (P + 4, P, P2, 2, 8, P3, None), (P, P, P2 + 2, 2, 8, P3, None),
    (P, P, P2, 2, 8, None, None),
])
def test_nft_noise_rejects(lib, args):
    assert fq.fp4_nft_noise(*args) == fq.binding.INVALID_ARGUMENT


def nl(**kw):
    a = dict(vo=P, vt=P, x0=P2, eps=P3, r=P, beta=0.5, n=2, d=8, partials=P2, terms=P3, loss=P, stream=None)
    a.update(kw)
    return fq.fp4_nft_loss(*a.values())


@pytest.mark.parametrize("kw", [
    dict(vo=None), dict(r=None), dict(partials=None), dict(loss=None), dict(n=0), dict(n=65536), dict(d=2),
    dict(d=10), dict(vt=P + 8), dict(r=P + 2), dict(beta=float("nan")), dict(beta=float("inf")),
])
def test_nft_loss_rejects(lib, kw):
    assert nl(**kw) == fq.binding.INVALID_ARGUMENT


def gern(**kw):
    a = dict(fmt=0, a=P, a_s=P3, b=P2, b_s=P3, m=256, n=256, k=64, residual=P2, x=P3, x_out=P, ldx=256,
             t_cur=1.0, t_next=5.0 / 6.0, u=P2, rows_per_cand=128, rewards=P, stream=None)
    a.update(kw)
    return fq.fp4_gemm_panel_euler_reward_noalloc(*a.values())


@pytest.mark.parametrize("kw", [
    dict(fmt=3), dict(a=None), dict(residual=None), dict(x=None), dict(x_out=None), dict(u=None), dict(u=P2 + 4),
    dict(rewards=None), dict(rewards=P + 1), dict(rows_per_cand=0), dict(rows_per_cand=96), dict(m=0), dict(k=48),
    dict(ldx=250), dict(x=P3 + 4),
    # the library-owned partial sums hold (m / 256) (n / 256) 4 <= 2^18 floats
    dict(m=256 * 512, n=256 * 129, ldx=256 * 129), dict(m=256 * 65537, n=256, ldx=256),
])
def test_gemm_panel_euler_reward_noalloc_rejects(lib, kw):
    assert gern(**kw) == fq.binding.INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(fmt=1), dict(m=384, rows_per_cand=128), dict(n=128, ldx=128),
                                dict(rows_per_cand=64)])
def test_gemm_panel_euler_reward_noalloc_unsupported(lib, kw):
    assert gern(**kw) == fq.binding.UNSUPPORTED
