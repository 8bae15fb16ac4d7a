"""Pins for the oracle's Euler step, proxy reward, normalisation and
selection (CPU only)."""
import itertools
import json
import os

import numpy as np

from oracle import euler, reward, rollout

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_schedule():
    t = euler.schedule(6)
    assert len(t) == 7 and t[0] == 1.0 and t[-1] == 0.0
    assert all(a > b for a, b in zip(t, t[1:]))


def test_euler_dt_zero_and_v_zero():
    rng = np.random.default_rng(14)
    x = rng.standard_normal(100).astype(np.float32)
    v = rng.standard_normal(100).astype(np.float32)
    np.testing.assert_array_equal(euler.step(x, v, np.float32(0.5), np.float32(0.5)), x)
    np.testing.assert_array_equal(euler.step(x, np.zeros_like(v), np.float32(1), np.float32(0.5)), x)


def test_constant_field_closed_form():
    """Euler is exact on a constant field: 6 steps from t=1 to 0 move x by -c."""
    x0 = np.array([0.25, -3.0, 10.0])
    c = np.array([1.0, 2.0, -0.5])
    t = euler.schedule(6)
    x = x0.copy()
    for i in range(6):
        x = euler.step(x, c, t[i], t[i + 1])
    np.testing.assert_allclose(x, x0 - c, rtol=0, atol=1e-7)


def test_linear_field_closed_form_sign_of_dt():
    """v = x: each step multiplies by (1 + dt) with dt = -1/6 -> (5/6)^6."""
    t = euler.schedule(6)
    x = np.array([1.0, -2.0])
    for i in range(6):
        x = euler.step(x, x, t[i], t[i + 1])
    np.testing.assert_allclose(x, np.array([1.0, -2.0]) * (5 / 6) ** 6, rtol=1e-6)


def test_proxy_reward_hand_cases():
    x = np.array([[1, 2], [3, 4], [10, 10], [10, 10]], dtype=np.float32)
    np.testing.assert_allclose(reward.proxy_reward(x, 2), [2.5, 10.0])
    u = np.array([1.0, -1.0])
    np.testing.assert_allclose(reward.proxy_reward(x, 2, u), [-1.0, 0.0])


def test_normalize_hand_cases():
    r = reward.normalize([1.0, 2.0, 3.0, 4.0])
    sd = np.sqrt(1.25)
    np.testing.assert_allclose(r, [0.0, 0.5 - 0.25 / sd, 0.5 + 0.25 / sd, 1.0], rtol=1e-15)
    assert np.all(reward.normalize([5.0, 5.0, 5.0]) == 0.5)
    r = reward.normalize(np.random.default_rng(0).standard_normal(50))
    assert r.min() >= 0 and r.max() <= 1


def test_normalize_monotone():
    x = np.random.default_rng(1).standard_normal(200)
    r = reward.normalize(x)
    o = np.argsort(x)
    assert np.all(np.diff(r[o]) >= 0)


def test_selection_golden():
    with open(os.path.join(GOLD, "selection.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        top, bottom = reward.select(np.array(c["r"], dtype=np.float64), c["k_top"], c["k_bottom"])
        assert top.tolist() == c["top"] and bottom.tolist() == c["bottom"], c


def rank_by_count(r):
    """Position of each index in the total order, by counting (no sort)."""
    n = len(r)
    return [sum(1 for j in range(n) if r[j] > r[i] or (r[j] == r[i] and j < i)) for i in range(n)]


def test_selection_against_rank_by_count():
    rng = np.random.default_rng(15)
    for trial in range(30):
        n = int(rng.integers(1, 40))
        r = rng.integers(-3, 4, n).astype(np.float64) if trial % 2 else rng.standard_normal(n)
        kt = int(rng.integers(0, n + 1))
        kb = int(rng.integers(0, n - kt + 1))
        top, bottom = reward.select(r, kt, kb)
        rank = rank_by_count(list(r))
        want_top = [None] * kt
        want_bottom = [None] * kb
        for i, p in enumerate(rank):
            if p < kt:
                want_top[p] = i
            if p >= n - kb:
                want_bottom[n - 1 - p] = i
        assert top.tolist() == want_top and bottom.tolist() == want_bottom
        assert not set(top.tolist()) & set(bottom.tolist())


def test_selection_permutation_equivariance():
    r = np.random.default_rng(16).standard_normal(96)      # distinct values
    top, bottom = reward.select(r, 12, 12)
    perm = np.random.default_rng(17).permutation(96)
    t2, b2 = reward.select(r[perm], 12, 12)
    np.testing.assert_array_equal(perm[t2], top)
    np.testing.assert_array_equal(perm[b2], bottom)


def test_rollout_zero_weights_closed_form():
    """With all weights zero the velocity is x itself, so 6 Euler steps give
    x0 (5/6)^6 -- through both the quantized and the unquantized linears."""
    rng = np.random.default_rng(18)
    noise = rng.standard_normal((3, 4, 32)).astype(np.float32)
    w1 = [np.zeros((64, 32), dtype=np.float32)] * 2
    w2 = [np.zeros((32, 64), dtype=np.float32)] * 2
    u = rng.standard_normal(32).astype(np.float32)
    for fmt in ("mx", "nv", None):
        x, r, top, bottom = rollout.rollout(noise, w1, w2, u, fmt=fmt, k_top=1, k_bottom=1)
        np.testing.assert_allclose(x, noise * (5 / 6) ** 6, rtol=1e-6)
        np.testing.assert_allclose(r, noise.mean(axis=1) @ u * (5 / 6) ** 6, rtol=1e-5)


def test_rollout_small_is_deterministic_and_ranks_agree():
    """Determinism, and a sanity property of the composite (its exact
    pins are in test_oracle_velocity_hand.py): the FP4 rollout's ranking
    should mostly agree with the unquantized one on a tiny problem."""
    rng = np.random.default_rng(19)
    noise = rng.standard_normal((8, 16, 64)).astype(np.float32)
    w1 = [(rng.standard_normal((128, 64)) * 0.02).astype(np.float32) for _ in range(2)]
    w2 = [(rng.standard_normal((64, 128)) * 0.02).astype(np.float32) for _ in range(2)]
    u = rng.standard_normal(64).astype(np.float32)
    a = rollout.rollout(noise, w1, w2, u, fmt="mx", k_top=2, k_bottom=2)
    b = rollout.rollout(noise, w1, w2, u, fmt="mx", k_top=2, k_bottom=2)
    np.testing.assert_array_equal(a[1], b[1])
    c = rollout.rollout(noise, w1, w2, u, fmt=None, k_top=2, k_bottom=2)
    # Spearman correlation of the two reward vectors
    ra, rc = np.argsort(np.argsort(a[1])), np.argsort(np.argsort(c[1]))
    rho = np.corrcoef(ra, rc)[0, 1]
    assert rho > 0.8


def test_selection_order_with_non_finite_rewards():
    """The order is total for any float: +inf first, then finite values by
    value (-0 ties with +0, by index), -inf, and every NaN last by index.
    Hand-worked: r = [nan, 1, -inf, inf, nan, -0.0, 0.0, -2]."""
    r = np.array([np.nan, 1.0, -np.inf, np.inf, np.nan, -0.0, 0.0, -2.0])
    assert reward.order(r) == [3, 1, 5, 6, 7, 2, 0, 4]
    top, bottom = reward.select(r, 3, 4)
    assert top.tolist() == [3, 1, 5] and bottom.tolist() == [4, 0, 2, 7]
