"""Pins of the DiffusionNFT oracle against values fixed by its equations
(VeRL-Omni DiffusionNFT docs, "Algorithm"), not by re-calling the oracle:

  * exact rational arithmetic with explicit loops on a tiny batch, where a
    swapped branch, a wrong sign of beta or a missing (1 - r) shows;
  * beta = 0: both branches equal v_old, so the loss is ||v_old - v||^2
    whatever r;
  * r = 1 keeps only the positive branch and r = 0 only the negative one;
  * v_theta = v_old: both branches equal v_old for every beta;
  * the noising path at t = 0 and t = 1 returns x0 and eps, and its time
    derivative (a finite difference, exact for a linear path) is the target
    velocity eps - x0.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import nft


def exact_terms(vo, vt, x0, eps, r, beta):
    out = []
    b = Fraction(float(beta))
    for i in range(vo.shape[0]):
        pos = neg = Fraction(0)
        for j in range(vo.shape[1]):
            v = Fraction(float(eps[i, j])) - Fraction(float(x0[i, j]))
            o, th = Fraction(float(vo[i, j])), Fraction(float(vt[i, j]))
            vp = (1 - b) * o + b * th
            vn = (1 + b) * o - b * th
            pos += (vp - v) ** 2
            neg += (vn - v) ** 2
        ri = Fraction(float(r[i]))
        out.append(ri * pos + (1 - ri) * neg)
    return out


def rand(seed, n=3, d=5):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((n, d)).astype(np.float32) for _ in range(4)] + [rng.uniform(0, 1, n)]


@pytest.mark.parametrize("seed,beta", [(0, 0.1), (1, 1.0), (2, 0.37)])
def test_against_exact_rationals(seed, beta):
    vo, vt, x0, eps, r = rand(seed)
    got = nft.loss_terms(vo, vt, x0, eps, r, beta)
    want = exact_terms(vo, vt, x0, eps, r, beta)
    for g, w in zip(got, want):
        assert abs(Fraction(float(g)) - w) <= Fraction(1e-12) * (1 + abs(w))


def test_beta_zero_is_plain_regression():
    vo, vt, x0, eps, r = rand(3)
    v = eps.astype(np.float64) - x0
    want = ((vo - v) ** 2).sum(axis=1)
    np.testing.assert_allclose(nft.loss_terms(vo, vt, x0, eps, r, 0.0), want, rtol=1e-14)


def test_r_selects_the_branch():
    vo, vt, x0, eps, _ = (a.astype(np.float64) for a in rand(4))
    beta = 0.5
    v = eps - x0
    pos = (((1 - beta) * vo + beta * vt - v) ** 2).sum(axis=1)
    neg = (((1 + beta) * vo - beta * vt - v) ** 2).sum(axis=1)
    np.testing.assert_allclose(nft.loss_terms(vo, vt, x0, eps, np.ones(3), beta), pos, rtol=1e-14)
    np.testing.assert_allclose(nft.loss_terms(vo, vt, x0, eps, np.zeros(3), beta), neg, rtol=1e-14)


def test_equal_velocities_make_beta_irrelevant():
    vo, _, x0, eps, r = rand(5)
    a = nft.loss_terms(vo, vo, x0, eps, r, 0.0)
    for beta in (0.3, 1.0, 2.5):
        np.testing.assert_allclose(nft.loss_terms(vo, vo, x0, eps, r, beta), a, rtol=1e-14)


def test_noising_path_and_velocity():
    _, _, x0, eps, _ = rand(6)
    np.testing.assert_array_equal(nft.noise(x0, eps, np.zeros(3)), x0)
    np.testing.assert_array_equal(nft.noise(x0, eps, np.ones(3)), eps)
    h = 0.25
    t = np.full(3, 0.5)
    fd = (nft.noise(x0, eps, t + h) - nft.noise(x0, eps, t - h)) / (2 * h)
    np.testing.assert_allclose(fd, nft.target_velocity(x0, eps), rtol=1e-12, atol=1e-12)
