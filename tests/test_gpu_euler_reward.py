"""GPU parity: euler_step, fp4_proxy_reward, select_topk_bottomk, and the
tiny end-to-end configuration (quantize -> GEMM -> reward -> selection)."""
import numpy as np
import pytest
import torch

from fp4_quantized_diffusion_amd import inputs
from oracle import euler as oeuler, gemm as ogemm, reward as oreward
from tests._parity import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("vdt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("numel", [1, 7, 1000003, 1 << 22])
def test_euler_step(gpu_lib, vdt, numel):
    rng = np.random.default_rng(numel)
    x = rng.standard_normal(numel).astype(np.float32)
    v = rng.standard_normal(numel).astype(np.float32)
    if vdt == torch.bfloat16:
        v = inputs.to_bf16(v)
    t = oeuler.schedule(6)
    xd, vd = dev(x), dev(v).to(vdt)
    out = to_np(gpu_lib.euler(xd, vd, t[1], t[2]))
    want = oeuler.step(x, v, t[1], t[2])
    dt = np.float64(t[2]) - np.float64(t[1])
    assert np.all(np.abs(out - want) <= 1e-3 * (np.abs(x) + np.abs(dt * v)) + 1e-30)
    gpu_lib.euler(xd, vd, t[1], t[2], out=xd)  # in place
    np.testing.assert_array_equal(to_np(xd), out)


def test_euler_dt_zero_copies_and_constant_field(gpu_lib):
    rng = np.random.default_rng(40)
    x = rng.standard_normal(4099).astype(np.float32)
    v = rng.standard_normal(4099).astype(np.float32)
    xd = dev(x)
    np.testing.assert_array_equal(to_np(gpu_lib.euler(xd, dev(v), 0.5, 0.5)), x)
    c = np.float32(0.75)
    cd = torch.full_like(xd, float(c))
    t = oeuler.schedule(6)
    for i in range(6):
        gpu_lib.euler(xd, cd, t[i], t[i + 1], out=xd)
    err = np.abs(to_np(xd).astype(np.float64) - (x.astype(np.float64) - float(c)))
    assert np.all(err <= 4e-7 * (np.abs(x) + 1)), float(err.max())


def test_proxy_reward_tiny_and_dot(gpu_lib):
    rng = np.random.default_rng(41)
    c = rng.standard_normal((128, 512)).astype(np.float32)
    r = to_np(gpu_lib.proxy_reward(dev(c), 8, 16))
    np.testing.assert_allclose(r, oreward.proxy_reward(c, 16), rtol=1e-5, atol=1e-7)
    x = rng.standard_normal((6 * 300, 256)).astype(np.float32)
    u = rng.standard_normal(256).astype(np.float32)
    r = to_np(gpu_lib.proxy_reward(dev(x), 6, 300, u=dev(u)))
    want = oreward.proxy_reward(x, 300, u)
    assert np.all(np.abs(r - want) <= 1e-5 * (np.abs(x).reshape(6, -1).mean(1) * np.abs(u).sum()))


@pytest.mark.parametrize("n,kt,kb,kind", [(96, 12, 12, "normal"), (8, 2, 2, "normal"), (96, 12, 12, "ties"),
                                          (1, 1, 0, "normal"), (5000, 100, 37, "ties"), (65536, 12, 12, "normal"),
                                          (10, 0, 10, "ties")])
def test_select_bit_exact(gpu_lib, n, kt, kb, kind):
    r = inputs.rewards(n, n, kind)
    top, bottom, rn = gpu_lib.select(dev(r), kt, kb)
    ot, ob = oreward.select(r, kt, kb)
    np.testing.assert_array_equal(to_np(top), ot)
    np.testing.assert_array_equal(to_np(bottom), ob)
    np.testing.assert_allclose(to_np(rn), oreward.normalize(r), rtol=0, atol=1e-5)


def test_select_all_equal(gpu_lib):
    r = np.full(12, 3.5, np.float32)
    top, bottom, rn = gpu_lib.select(dev(r), 3, 4)
    assert to_np(top).tolist() == [0, 1, 2] and to_np(bottom).tolist() == [11, 10, 9, 8]
    assert np.all(to_np(rn) == 0.5)


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_tiny_config_end_to_end(gpu_lib, fmt):
    """Tiny configuration: quantize X and W, GEMM (fp32), rewards = mean of
    16-row slices, top-2 / bottom-2. The selection must match the oracle's
    unless two rewards straddling the cut are closer than the GEMM error
    bound allows to separate."""
    x, b = inputs.tiny(0)
    qa = gpu_lib.quantize(dev(x), fmt)
    qb = gpu_lib.quantize(dev(b), fmt)
    c = gpu_lib.gemm(qa, qb, "f32")
    r = gpu_lib.proxy_reward(c, 8, 16)
    top, bottom, rn = gpu_lib.select(r, 2, 2)
    k = 256
    if fmt == "mx":
        c_exact, s_abs = ogemm.gemm_mx(to_np(qa.codes)[:, :k // 2], to_np(qa.scales),
                                       to_np(qb.codes)[:, :k // 2], to_np(qb.scales))
    else:
        c_exact, s_abs = ogemm.gemm_nv(to_np(qa.codes)[:, :k // 2], to_np(qa.scales), to_np(qa.tensor_scale)[0],
                                       to_np(qb.codes)[:, :k // 2], to_np(qb.scales), to_np(qb.tensor_scale)[0])
    r_or = oreward.proxy_reward(c_exact, 16)
    bound = (1e-4 * s_abs).reshape(8, -1).mean(1) + 1e-6 * np.abs(r_or)
    np.testing.assert_allclose(to_np(r), r_or, rtol=0, atol=float(bound.max()) * 2)
    ot, ob = oreward.select(r_or, 2, 2)
    order = oreward.order(r_or)
    gaps = np.abs(np.diff(np.asarray(r_or)[order]))
    if gaps.min() > 4 * bound.max():
        np.testing.assert_array_equal(to_np(top), ot)
        np.testing.assert_array_equal(to_np(bottom), ob)
    else:
        # near-tie: the GPU's choice must be a valid selection of its own rewards
        gt, gb = oreward.select(to_np(r), 2, 2)
        np.testing.assert_array_equal(to_np(top), gt)
        np.testing.assert_array_equal(to_np(bottom), gb)


@pytest.mark.parametrize("n,kt,kb", [(8, 3, 4), (96, 12, 12), (300, 40, 50)])
def test_select_non_finite_rewards(gpu_lib, n, kt, kb):
    """NaN and infinite rewards still give a permutation: every requested slot
    holds a valid index, equal to the oracle's total order (NaN below -inf,
    -0 equal to +0). The output buffers start as sentinels, so an unwritten
    slot would show."""
    import torch
    rng = np.random.default_rng(n)
    r = rng.standard_normal(n).astype(np.float32)
    special = np.array([np.nan, np.inf, -np.inf, -0.0, 0.0, np.nan, 1.0, -np.inf], np.float32)
    pos = rng.choice(n, size=min(n, len(special)), replace=False)
    r[pos] = special[:len(pos)]
    top = torch.full((kt,), -7, dtype=torch.int32, device=DEV)
    bottom = torch.full((kb,), -7, dtype=torch.int32, device=DEV)
    from fp4_quantized_diffusion_amd import binding as fb
    rd = dev(r)
    st = fb.select_topk_bottomk(rd.data_ptr(), n, kt, kb, top.data_ptr(), bottom.data_ptr(), None,
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0
    ot, ob = oreward.select(r, kt, kb)
    np.testing.assert_array_equal(to_np(top), ot)
    np.testing.assert_array_equal(to_np(bottom), ob)
