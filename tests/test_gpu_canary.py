"""Canary checks of every output buffer: each call writes into a region of a
larger buffer that is filled with a sentinel first -- row padding past the
logical width (ld > width), rows past the last one, bytes past the end of a
panel-layout or vector output -- and afterwards every sentinel must be
intact. Ragged sizes make the kernels take their edge paths. The values
written inside the region are checked against the oracle elsewhere; here only
what lies outside it is."""
import numpy as np
import pytest
import torch

import fp4_quantized_diffusion_amd as fq
from fp4_quantized_diffusion_amd import binding as fb
from tests._parity import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
S32 = -0x4546B3DB  # 0xBAB94C25 as int32: a distinctive fp32 bit pattern
S16 = -0x4547      # 0xBAB9 as int16
S8 = 0xA5


def canvas(rows, cols, dtype):
    """A [rows, cols] buffer of sentinel bits."""
    if dtype == torch.float32:
        return torch.full((rows, cols), S32, dtype=torch.int32, device=DEV).view(torch.float32)
    if dtype == torch.bfloat16:
        return torch.full((rows, cols), S16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    return torch.full((rows, cols), S8, dtype=torch.uint8, device=DEV)


def untouched(t):
    """True where t still holds the sentinel bits."""
    if t.dtype == torch.float32:
        return t.view(torch.int32) == S32
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16) == S16
    return t == S8


def assert_outside_intact(buf, rows, cols, what):
    assert bool(untouched(buf[:rows, cols:]).all()), f"{what}: row padding written"
    assert bool(untouched(buf[rows:]).all()), f"{what}: rows past the end written"


def rand_q(rows, k, fmt, layout="row", seed=0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randn(rows, k, device=DEV, generator=g)
    return fq.quantize(x, fmt, layout=layout)


@pytest.mark.parametrize("fmt,layout", [("mx", "row"), ("nv", "row"), ("mx", "panel")])
@pytest.mark.parametrize("out_dtype,resid", [("f32", False), ("f32", True), ("bf16", False)])
@pytest.mark.parametrize("m,n,k", [(300, 200, 96), (513, 260, 384), (17, 5, 32)])
def test_gemm_writes_only_its_output(gpu_lib, fmt, layout, out_dtype, resid, m, n, k):
    if fmt == "nv" and k % 16:
        pytest.skip("k")
    qa, qb = rand_q(m, k, fmt, layout, 1), rand_q(n, k, fmt, layout, 2)
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    ldc = (n + 3) // 4 * 4 + 12
    buf = canvas(m + 5, ldc, dt)
    out = buf[:m, :n]
    residual = None
    if resid:
        rbuf = torch.randn(m, ldc, device=DEV)
        residual = rbuf[:, :n]
    fq.gemm(qa, qb, out_dtype, residual=residual, out=out)
    torch.cuda.synchronize()
    if dt == torch.float32:  # (a bf16 result may hit the 16-bit sentinel by chance)
        assert not bool(untouched(out).any()), "output not fully written"
    assert_outside_intact(buf, m, n, f"gemm {fmt} {layout} {out_dtype}")


@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("rows,k", [(37, 96), (300, 512), (1, 32)])
def test_quantize_row_layout_writes_only_its_output(gpu_lib, fmt, rows, k):
    blk = 32 if fmt == "mx" else 16
    x = torch.randn(rows, k, device=DEV)
    ldcodes = k // 2 + 12
    ldsc = k // blk + 3
    cb, sb = canvas(rows + 3, ldcodes, torch.uint8), canvas(rows + 3, ldsc, torch.uint8)
    ts = torch.empty(1, dtype=torch.float32, device=DEV) if fmt == "nv" else None
    out = fb.QTensor(cb[:rows], sb[:rows, : k // blk], ts, fb.FMT_MX if fmt == "mx" else fb.FMT_NV, k)
    fq.quantize(x, fmt, out=out)
    torch.cuda.synchronize()
    assert_outside_intact(cb, rows, k // 2, f"{fmt} codes")
    assert_outside_intact(sb, rows, k // blk, f"{fmt} scales")


@pytest.mark.parametrize("prologue", [None, "rmsnorm", "gelu"])
@pytest.mark.parametrize("rows,k", [(300, 160), (256, 4224)])
def test_quantize_panel_writes_only_its_output(gpu_lib, prologue, rows, k):
    x = torch.randn(rows, k, device=DEV)
    cbytes, sbytes = fb.panel_bytes(rows, k)
    cb, sb = canvas(1, cbytes + 4096, torch.uint8)[0], canvas(1, sbytes + 256, torch.uint8)[0]
    out = fb.QTensor(cb[:cbytes], sb[:sbytes], None, fb.FMT_MX, k, "panel", rows)
    fq.quantize(x, "mx", prologue=prologue, out=out)
    torch.cuda.synchronize()
    assert bool(untouched(cb[cbytes:]).all()) and bool(untouched(sb[sbytes:]).all())
    assert not bool(untouched(sb[:sbytes]).all())


def test_fused_gemms_write_only_their_outputs(gpu_lib):
    """The GELU + MXFP4 epilogue (panel codes and scales), the Euler epilogue
    (state with ldx > n) and the Euler + reward epilogue (rewards and its
    partial-sum workspace)."""
    m, n, k, hidden = 512, 256, 256, 512
    qa = rand_q(m, k, "mx", "panel", 3)
    w1, w2 = rand_q(hidden, k, "mx", "panel", 4), rand_q(n, hidden, "mx", "panel", 5)
    cbytes, sbytes = fb.panel_bytes(m, hidden)
    cb, sb = canvas(1, cbytes + 4096, torch.uint8)[0], canvas(1, sbytes + 256, torch.uint8)[0]
    a2 = fb.QTensor(cb[:cbytes], sb[:sbytes], None, fb.FMT_MX, hidden, "panel", m)
    fq.gemm_gelu(qa, w1, out=a2)
    ldx = n + 16
    x = torch.randn(m, ldx, device=DEV)[:, :n]
    resid = torch.randn(m, ldx, device=DEV)[:, :n]
    xbuf = canvas(m + 3, ldx, torch.float32)
    fq.gemm_euler(a2, w2, resid, x, 1.0, 5.0 / 6.0, out=xbuf[:m, :n])
    rbuf = canvas(1, 8, torch.float32)[0]
    need = (m // 256) * (n // 256) * 4
    pbuf = canvas(1, need + 64, torch.float32)[0]
    u = torch.randn(n, device=DEV)
    xbuf2 = canvas(m + 3, ldx, torch.float32)
    fq.gemm_euler_reward(a2, w2, resid, x, 1.0, 5.0 / 6.0, u, 256, out=xbuf2[:m, :n], rewards=rbuf[:2],
                         partials=pbuf[:need])
    torch.cuda.synchronize()
    assert bool(untouched(cb[cbytes:]).all()) and bool(untouched(sb[sbytes:]).all())
    assert_outside_intact(xbuf, m, n, "euler epilogue")
    assert_outside_intact(xbuf2, m, n, "euler + reward epilogue")
    assert bool(untouched(rbuf[2:]).all()) and not bool(untouched(rbuf[:2]).any())
    assert bool(untouched(pbuf[need:]).all())


@pytest.mark.parametrize("numel", [1, 7, 1001, 1 << 20 | 3])
@pytest.mark.parametrize("vdt", [torch.float32, torch.bfloat16])
def test_euler_writes_only_its_output(gpu_lib, numel, vdt):
    x = torch.randn(numel, device=DEV)
    v = torch.randn(numel, device=DEV).to(vdt)
    buf = canvas(1, numel + 37, torch.float32)[0]
    fq.euler(x, v, 1.0, 5.0 / 6.0, out=buf[:numel])
    torch.cuda.synchronize()
    assert bool(untouched(buf[numel:]).all())
    want = x + (np.float32(5.0 / 6.0) - np.float32(1.0)) * v.float()
    assert torch.allclose(buf[:numel], want, rtol=1e-6, atol=1e-6)


def test_reward_and_select_write_only_their_outputs(gpu_lib):
    n_cand, rows, dim = 6, 100, 192
    x = torch.randn(n_cand * rows, dim, device=DEV)
    rbuf = canvas(1, n_cand + 9, torch.float32)[0]
    fq.proxy_reward(x, n_cand, rows, u=torch.randn(dim, device=DEV), out=rbuf[:n_cand])
    tb = torch.full((8,), -7, dtype=torch.int32, device=DEV)
    bb = torch.full((8,), -7, dtype=torch.int32, device=DEV)
    nb = canvas(1, n_cand + 5, torch.float32)[0]
    st = fb.select_topk_bottomk(rbuf.data_ptr(), n_cand, 2, 3, tb.data_ptr(), bb.data_ptr(), nb.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert bool(untouched(rbuf[n_cand:]).all())
    assert to_np(tb[2:]).tolist() == [-7] * 6 and to_np(bb[3:]).tolist() == [-7] * 5
    assert bool(untouched(nb[n_cand:]).all()) and not bool(untouched(nb[:n_cand]).any())
