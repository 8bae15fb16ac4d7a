"""GPU parity of the DiffusionNFT pieces (fp4_nft_noise, fp4_nft_loss)
against the float64 oracle (oracle/nft.py):

  * noising: within one fp32 rounding of each of its three operations of
    the exact path value;
  * loss terms: within the fp32 summation bound (count + 6) 2^-24 times the
    sum of the magnitudes involved, per sample and for the mean; r = 0 and
    r = 1 select one branch; beta = 0 makes the terms independent of
    v_theta (bit for bit); repeated calls give the same bits;
  * the regenerated-sample shape (4096 x 3072 values per sample).
"""
import numpy as np
import pytest
import torch

from oracle import nft
from tests._parity import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def arrays(n, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((n, d)).astype(np.float32) for _ in range(4)]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("n,d", [(1, 4), (3, 1000), (24, 4096)])
def test_noise(gpu_lib, n, d):
    x0, eps, _, _ = arrays(n, d, n + d)
    t = np.random.default_rng(d).uniform(0, 1, n).astype(np.float32)
    got = to_np(gpu_lib.nft_noise(dev(x0), dev(eps), dev(t))).astype(np.float64)
    want = nft.noise(x0, eps, t)
    mag = np.abs(x0) * (1 - t[:, None]) + np.abs(eps) * t[:, None]
    assert (np.abs(got - want) <= 3 * 2.0 ** -24 * mag + 1e-45).all()


def loss_bound(vo, vt, x0, eps, beta, d):
    v = eps.astype(np.float64) - x0
    a = np.abs((1 - beta) * vo.astype(np.float64)) + np.abs(beta * vt.astype(np.float64)) + np.abs(v)
    b = np.abs((1 + beta) * vo.astype(np.float64)) + np.abs(beta * vt.astype(np.float64)) + np.abs(v)
    return (d + 12) * 2.0 ** -24 * ((a ** 2).sum(axis=1) + (b ** 2).sum(axis=1))


@pytest.mark.parametrize("n,d,beta", [(2, 8, 0.5), (5, 3000, 1.0), (24, 12288, 0.1), (1, 65536, 2.0)])
def test_loss_against_oracle(gpu_lib, n, d, beta):
    vo, vt, x0, eps = arrays(n, d, n * d)
    r = np.random.default_rng(n).uniform(0, 1, n).astype(np.float32)
    loss, terms = gpu_lib.nft_loss(dev(vo), dev(vt), dev(x0), dev(eps), dev(r), beta)
    want = nft.loss_terms(vo, vt, x0, eps, r, beta)
    bound = loss_bound(vo, vt, x0, eps, beta, d)
    assert (np.abs(to_np(terms) - want) <= bound).all()
    assert abs(float(to_np(loss)[0]) - want.mean()) <= bound.mean() + 2.0 ** -23 * abs(want.mean()) * (n + 2)


def test_branch_selection_and_beta_zero(gpu_lib):
    n, d = 4, 2048
    vo, vt, x0, eps = arrays(n, d, 9)
    ones, zeros = np.ones(n, np.float32), np.zeros(n, np.float32)
    _, tp = gpu_lib.nft_loss(dev(vo), dev(vt), dev(x0), dev(eps), dev(ones), 0.5)
    _, tn = gpu_lib.nft_loss(dev(vo), dev(vt), dev(x0), dev(eps), dev(zeros), 0.5)
    bound = loss_bound(vo, vt, x0, eps, 0.5, d)
    assert (np.abs(to_np(tp) - nft.loss_terms(vo, vt, x0, eps, ones, 0.5)) <= bound).all()
    assert (np.abs(to_np(tn) - nft.loss_terms(vo, vt, x0, eps, zeros, 0.5)) <= bound).all()
    r = dev(np.random.default_rng(1).uniform(0, 1, n).astype(np.float32))
    _, t1 = gpu_lib.nft_loss(dev(vo), dev(vt), dev(x0), dev(eps), r, 0.0)
    _, t2 = gpu_lib.nft_loss(dev(vo), dev(-3 * vt), dev(x0), dev(eps), r, 0.0)
    np.testing.assert_array_equal(to_np(t1), to_np(t2))
    _, t3 = gpu_lib.nft_loss(dev(vo), dev(vt), dev(x0), dev(eps), r, 0.0)
    np.testing.assert_array_equal(to_np(t1), to_np(t3))


def test_regenerated_sample_shape(gpu_lib):
    """Two samples of 4096 x 3072 values (a regenerated latent's size)."""
    n, d = 2, 4096 * 3072
    vo, vt, x0, eps = arrays(n, d, 2)
    r = np.array([0.2, 0.9], np.float32)
    loss, terms = gpu_lib.nft_loss(dev(vo), dev(vt), dev(x0), dev(eps), dev(r), 0.1)
    want = nft.loss_terms(vo, vt, x0, eps, r, 0.1)
    assert (np.abs(to_np(terms) - want) <= loss_bound(vo, vt, x0, eps, 0.1, d)).all()
