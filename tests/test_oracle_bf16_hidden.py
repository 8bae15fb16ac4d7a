"""Pins of the oracle's second reading of the hidden activation
(oracle.rollout, hidden="bf16": z rounded to fp32 and then to bf16, nearest
even, before GELU):
  * bf16_round against torch's CPU casts (float64 -> float32 -> bfloat16,
    each nearest-even) over every binade, exact ties with both parities of
    the kept bit, near-ties, overflow to infinity, zeros and subnormals;
  * the hand-worked block of tests/golden/velocity_bf16_hidden.json, where
    the two readings give different exact outputs, and the wrong tensor
    rounded (the GELU output or the RMSNorm output instead of z) misses;
  * when every z is bf16-exact (tests/golden/velocity_hand.json) the two
    readings agree."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import mxfp4, rollout as orollout

GOLD_DIR = os.path.join(os.path.dirname(__file__), "golden")
G = json.load(open(os.path.join(GOLD_DIR, "velocity_bf16_hidden.json")))
HAND = json.load(open(os.path.join(GOLD_DIR, "velocity_hand.json")))


def torch_bf16(v64):
    t = torch.from_numpy(np.asarray(v64, dtype=np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def vec(spec, n=32):
    v = [Fraction(spec["fill"])] * n
    for i, val in spec["set"]:
        v[i] = Fraction(val)
    return np.array([float(f) for f in v])


def mat(entries, n=32):
    w = np.zeros((n, n), np.float32)
    for r, c, v in entries:
        w[r, c] = v
    return w


def test_bf16_round_matches_torch_over_binades():
    rng = np.random.default_rng(11)
    mant = rng.random(200000) + 1.0
    expo = rng.integers(-140, 128, 200000)
    sign = np.where(rng.random(200000) < 0.5, -1.0, 1.0)
    v = sign * np.ldexp(mant, expo)                       # float64, many not fp32-exact
    v = v[np.abs(v) < 3.3e38]
    np.testing.assert_array_equal(orollout.bf16_round(v), torch_bf16(v))


def test_bf16_round_ties_and_edges():
    rng = np.random.default_rng(12)
    hi = rng.integers(0, 0x7F7F, 50000, dtype=np.uint64) << 16             # bf16 patterns, both parities
    pats = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi, hi | 0xFFFF])
    pats = pats[(pats & 0x7F800000) != 0x7F800000]                            # finite fp32 only
    f = pats.astype(np.uint32).view(np.float32).astype(np.float64)
    f = np.concatenate([f, -f, [0.0, -0.0, 3.4028234663852886e38, 1.4e-45, -1.4e-45, 1.1754942e-38]])
    got, want = orollout.bf16_round(f), torch_bf16(f)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(want))       # -0 keeps its sign
    # ties go to the even kept pattern: 1 + 2^-8 (tie, kept bit 0) stays 1, 1 + 3 * 2^-8 goes up
    assert orollout.bf16_round(1 + 2 ** -8) == 1.0
    assert orollout.bf16_round(1 + 3 * 2 ** -8) == 1 + 2 ** -6


def test_hand_block_both_readings():
    x = np.array([vec(G["x"])], np.float32)
    l1, l2 = orollout.QuantLinear(mat(G["w1"]), "mx"), orollout.QuantLinear(mat(G["w2"]), "mx")
    for w in (mat(G["w1"]), mat(G["w2"])):
        assert np.array_equal(mxfp4.dequant(*mxfp4.quantize(w)), w)
    a = mxfp4.dequant(*mxfp4.quantize(orollout.rmsnorm(x).astype(np.float32)))
    np.testing.assert_array_equal(a[0], vec(G["a_hat"]))
    np.testing.assert_array_equal(l1(orollout.rmsnorm(x))[0], vec(G["z"]))
    for reading in ("f32", "bf16"):
        h = orollout.velocity(x, [l1], [l2], hidden=reading)
        np.testing.assert_array_equal(h[0], vec(G[reading]["h"]))


def test_hand_block_rounding_the_wrong_tensor_misses():
    """Rounding the GELU output, or the RMSNorm output, instead of z (built
    from the oracle's own pieces) gives the f32 reading's outputs here, not
    the bf16 reading's."""
    x = np.array([vec(G["x"])], np.float32)
    l1, l2 = orollout.QuantLinear(mat(G["w1"]), "mx"), orollout.QuantLinear(mat(G["w2"]), "mx")
    want = vec(G["bf16"]["h"])
    round_g = x + l2(orollout.bf16_round(orollout.gelu(l1(orollout.rmsnorm(x)))))
    round_y = x + l2(orollout.gelu(l1(orollout.bf16_round(orollout.rmsnorm(x)))))
    for h in (round_g, round_y):
        assert not np.array_equal(h[0], want)


@pytest.mark.parametrize("blocks", [1, 2])
def test_readings_agree_when_z_is_bf16_exact(blocks):
    w1, w2 = mat(HAND["w1"]), mat(HAND["w2"])
    x = np.array([vec(HAND["x"])], np.float32)
    l1, l2 = orollout.QuantLinear(w1, "mx"), orollout.QuantLinear(w2, "mx")
    a = orollout.velocity(x, [l1] * blocks, [l2] * blocks, hidden="f32")
    b = orollout.velocity(x, [l1] * blocks, [l2] * blocks, hidden="bf16")
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a[0], vec(HAND["block1" if blocks == 1 else "block2"]["h"]))


def test_unknown_reading_is_rejected():
    with pytest.raises(ValueError):
        orollout.velocity(np.zeros((1, 32), np.float32), [], [], hidden="f16")
