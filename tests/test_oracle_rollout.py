"""Pins of the rollout oracle's elementwise pieces against values fixed by
the mathematics (not by re-calling the oracle's own library routine):

GELU(z) = z Phi(z) with Phi the standard normal CDF --
  * Phi at integer points from the standard normal table;
  * the identity GELU(z) - GELU(-z) = z (Phi(z) + Phi(-z) = 1), which a sign
    or argument slip breaks;
  * the far negative tail against the asymptotic (Mills-ratio) series
    Phi(-z) = phi(z)/z * sum_n (-1)^n (2n-1)!! / z^(2n), whose error is below
    the first omitted term -- here relative accuracy is what the fused
    quantizer's codes depend on.
RMSNorm(h) = h / sqrt(mean(h^2) + 1e-6) --
  * a hand-worked row, constant rows, the zero row, and the mean-square
    identity mean(out^2) = ms / (ms + 1e-6)."""
import math

import numpy as np
import pytest

from oracle import rollout as orollout

# standard normal CDF at -1 .. -6, -8, -10 (table values)
PHI_TABLE = {
    1: 0.15865525393145705, 2: 0.022750131948179212, 3: 0.0013498980316300933,
    4: 3.1671241833119857e-05, 5: 2.866515718791939e-07, 6: 9.865876450377e-10,
    8: 6.22096057427178e-16, 10: 7.619853024160525e-24,
}


@pytest.mark.parametrize("z", sorted(PHI_TABLE))
def test_gelu_table_values(z):
    phi_neg = PHI_TABLE[z]
    assert orollout.gelu(-float(z)) == pytest.approx(-z * phi_neg, rel=1e-12)
    assert orollout.gelu(float(z)) == pytest.approx(z * (1.0 - phi_neg), rel=1e-14)


def test_gelu_zero_and_symmetry():
    assert orollout.gelu(0.0) == 0.0
    z = np.linspace(-9.0, 9.0, 2001)
    np.testing.assert_allclose(orollout.gelu(z) - orollout.gelu(-z), z, rtol=0, atol=1e-14)


def mills_tail(z, terms):
    """Phi(-z) from the asymptotic series and the size of its first omitted term."""
    phi = math.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    s, df = 0.0, 1.0  # (2n - 1)!!
    for n in range(terms):
        if n > 0:
            df *= 2 * n - 1
        s += (-1) ** n * df / z ** (2 * n)
    omitted = df * (2 * terms - 1) / z ** (2 * terms)
    return phi / z * s, phi / z * omitted


@pytest.mark.parametrize("z", [7.0, 8.0, 10.0, 12.0, 20.0, 30.0])
def test_gelu_negative_tail_relative_accuracy(z):
    ref, bound = mills_tail(z, 6)
    got = orollout.gelu(-z) / (-z)
    assert abs(got - ref) <= bound + 1e-12 * ref, (got, ref, bound)  # series bound + float64 rounding
    assert abs(got - ref) / ref < 1e-6


def test_rmsnorm_hand_row():
    out = orollout.rmsnorm(np.array([[3.0, 4.0]]))
    d = math.sqrt(12.5 + 1e-6)
    np.testing.assert_allclose(out, [[3.0 / d, 4.0 / d]], rtol=1e-15)


@pytest.mark.parametrize("c", [1e-4, 0.5, -2.0, 1e3])
def test_rmsnorm_constant_row(c):
    out = orollout.rmsnorm(np.full((1, 64), c))
    np.testing.assert_allclose(out, c / math.sqrt(c * c + 1e-6), rtol=1e-14)


def test_rmsnorm_zero_row_and_mean_square():
    assert (orollout.rmsnorm(np.zeros((2, 16))) == 0).all()
    h = np.random.default_rng(0).standard_normal((8, 3072)) * np.logspace(-4, 2, 8)[:, None]
    out = orollout.rmsnorm(h)
    ms = (h * h).mean(axis=1)
    np.testing.assert_allclose((out * out).mean(axis=1), ms / (ms + 1e-6), rtol=1e-13)
