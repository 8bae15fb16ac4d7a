"""GPU parity of NVFP4-style quantization with one tensor scale per group of
rows (fp4_quantize_nv_grouped) and of the GEMM that consumes it
(fp4_gemm_nv_grouped):

  * each group's codes, E4M3 scales and tensor scale equal those of an
    fp4_quantize(FP4_FMT_NV) call on that group alone, and the oracle's
    nvfp4.quantize of the group, bit for bit;
  * each group's rows of the grouped GEMM equal an fp4_gemm of that group
    alone, bit for bit (bf16 and fp32 out, with a residual), and are within
    the GEMM tolerance of the oracle with the group's tensor scale;
  * one group reproduces the ungrouped calls bit for bit; given scales are
    used as given.
Groups differ in magnitude by orders of ten, so a shared tensor scale would
change the codes of the small-magnitude groups."""
import numpy as np
import pytest
import torch

from oracle import gemm as ogemm, nvfp4
from tests._parity import gemm_within_tol, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def grouped_act(groups, rpg, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((groups, rpg, k)).astype(np.float32)
    x *= (10.0 ** rng.integers(-3, 3, size=groups)).astype(np.float32)[:, None, None]
    return x.reshape(groups * rpg, k)


@pytest.mark.parametrize("groups,rpg,k", [(4, 64, 256), (6, 300, 2432), (1, 128, 3072), (8, 1, 64)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_grouped_quantize_equals_per_group(gpu_lib, groups, rpg, k, dtype):
    x = grouped_act(groups, rpg, k, groups * rpg + k)
    xd = torch.from_numpy(x).to(DEV).to(dtype)
    q = gpu_lib.quantize_nv_grouped(xd, rpg)
    gc, gs, gts = to_np(q.codes)[:, : k // 2], to_np(q.scales)[:, : k // 16], to_np(q.tensor_scale)
    xr = xd.float().cpu().numpy()
    for g in range(groups):
        rows = slice(g * rpg, (g + 1) * rpg)
        p = gpu_lib.quantize(xd[rows], "nv")
        np.testing.assert_array_equal(gc[rows], to_np(p.codes)[:, : k // 2])
        np.testing.assert_array_equal(gs[rows], to_np(p.scales)[:, : k // 16])
        assert gts[g] == to_np(p.tensor_scale)[0]
        oc, os_, osg = nvfp4.quantize(xr[rows])
        np.testing.assert_array_equal(gc[rows], oc)
        np.testing.assert_array_equal(gs[rows], os_)
        assert np.float32(gts[g]) == np.float32(osg)


def test_grouped_quantize_given_scales(gpu_lib):
    groups, rpg, k = 3, 32, 128
    x = grouped_act(groups, rpg, k, 5)
    sg = np.array([0.5, 0.0625, 2.0], np.float32)
    q = gpu_lib.quantize_nv_grouped(torch.from_numpy(x).to(DEV), rpg, tensor_scales=torch.from_numpy(sg).to(DEV))
    np.testing.assert_array_equal(to_np(q.tensor_scale), sg)
    for g in range(groups):
        rows = slice(g * rpg, (g + 1) * rpg)
        oc, os_, _ = nvfp4.quantize(x[rows], s_g=sg[g])
        np.testing.assert_array_equal(to_np(q.codes)[rows, : k // 2], oc)
        np.testing.assert_array_equal(to_np(q.scales)[rows, : k // 16], os_)


@pytest.mark.parametrize("groups,rpg,n,k", [(4, 64, 256, 512), (3, 300, 200, 1024), (2, 256, 512, 3072)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_grouped_gemm_equals_per_group(gpu_lib, groups, rpg, n, k, out):
    x = grouped_act(groups, rpg, k, groups + rpg + n)
    rng = np.random.default_rng(n + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    xd = torch.from_numpy(x).to(DEV)
    qa = gpu_lib.quantize_nv_grouped(xd, rpg)
    qb = gpu_lib.quantize(torch.from_numpy(w).to(DEV), "nv")
    res = torch.from_numpy(rng.standard_normal((groups * rpg, n)).astype(np.float32)).to(DEV) if out == "f32" else None
    c = to_np(gpu_lib.gemm(qa, qb, out, residual=res).float())
    ts = to_np(qa.tensor_scale)
    bc, bs = to_np(qb.codes)[:, : k // 2], to_np(qb.scales)[:, : k // 16]
    for g in range(groups):
        rows = slice(g * rpg, (g + 1) * rpg)
        pa = gpu_lib.quantize(xd[rows], "nv")
        cg = to_np(gpu_lib.gemm(pa, qb, out, residual=None if res is None else res[rows]).float())
        np.testing.assert_array_equal(c[rows], cg)
        ce, s_abs = ogemm.gemm_nv(to_np(qa.codes)[rows, : k // 2], to_np(qa.scales)[rows, : k // 16], ts[g], bc, bs,
                                  to_np(qb.tensor_scale)[0])
        if res is not None:
            ce = ce + to_np(res[rows]).astype(np.float64)
        ok, worst = gemm_within_tol(c[rows], ce, s_abs, bf16_out=(out == "bf16"))
        assert ok, worst


def test_one_group_is_the_ungrouped_path(gpu_lib):
    rows, n, k = 256, 256, 1024
    rng = np.random.default_rng(1)
    xd = torch.from_numpy(rng.standard_normal((rows, k)).astype(np.float32)).to(DEV)
    wd = torch.from_numpy((rng.standard_normal((n, k)) * 0.02).astype(np.float32)).to(DEV)
    qg = gpu_lib.quantize_nv_grouped(xd, rows)
    qu = gpu_lib.quantize(xd, "nv")
    qb = gpu_lib.quantize(wd, "nv")
    np.testing.assert_array_equal(to_np(qg.codes), to_np(qu.codes))
    np.testing.assert_array_equal(to_np(qg.scales), to_np(qu.scales))
    np.testing.assert_array_equal(to_np(qg.tensor_scale), to_np(qu.tensor_scale))
    np.testing.assert_array_equal(to_np(gpu_lib.gemm(qg, qb, "f32")), to_np(gpu_lib.gemm(qu, qb, "f32")))
