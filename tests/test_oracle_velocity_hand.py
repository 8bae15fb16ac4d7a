"""Hand-worked pin of the oracle's composite velocity network and Euler step
(tests/golden/velocity_hand.json): one token, MXFP4-exact weights, inputs
whose quantization is far from every decision point, so the expected values
are exact rationals. A wrong block composition -- RMSNorm skipped or applied
after the first linear, GELU and RMSNorm exchanged, W1 and W2 exchanged, the
residual dropped, the second block fed the wrong state -- changes them; each
such variant is built from the oracle's own pieces below and must miss."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import mxfp4, rollout as orollout

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "velocity_hand.json")))


def vec(spec, n=32):
    v = [Fraction(spec["fill"])] * n
    for i, val in spec["set"]:
        v[i] = Fraction(val)
    return v


def mat(entries, n=32):
    w = np.zeros((n, n), np.float32)
    for r, c, v in entries:
        w[r, c] = v
    return w


def as_f64(frs):
    return np.array([float(f) for f in frs])


X = np.array([as_f64(vec(GOLD["x"]))], np.float32)
W1, W2 = mat(GOLD["w1"]), mat(GOLD["w2"])


def test_weights_are_mxfp4_exact():
    for w in (W1, W2):
        assert np.array_equal(mxfp4.dequant(*mxfp4.quantize(w)), w)


def test_quantized_activation_of_block1():
    """The first linear's input: RMSNorm(x) quantized (hand: [3, 1 x31])."""
    a = mxfp4.dequant(*mxfp4.quantize(orollout.rmsnorm(X).astype(np.float32)))
    assert np.array_equal(a[0], as_f64(vec(GOLD["block1"]["a_hat"])))


def test_one_block():
    l1, l2 = orollout.QuantLinear(W1, "mx"), orollout.QuantLinear(W2, "mx")
    h = orollout.velocity(X, [l1], [l2])
    assert np.array_equal(h[0], as_f64(vec(GOLD["block1"]["h"])))


def test_two_blocks():
    l1, l2 = orollout.QuantLinear(W1, "mx"), orollout.QuantLinear(W2, "mx")
    h = orollout.velocity(X, [l1, l1], [l2, l2])
    assert np.array_equal(h[0], as_f64(vec(GOLD["block2"]["h"])))


def test_one_euler_step_and_reward():
    u = np.zeros(32, np.float32)
    u[0] = 1.0
    xf, r, top, bottom = orollout.rollout(X[None], [W1], [W2], u, n_steps=1, fmt="mx", k_top=1, k_bottom=0)
    assert np.array_equal(xf[0, 0], as_f64(vec(GOLD["euler_one_step"]["x1"])))
    assert r[0] == GOLD["euler_one_step"]["reward"] and top.tolist() == [0]


def test_plausible_mistakes_miss_the_pin():
    """Variants of the block built from the oracle's own pieces: each must
    differ from the hand-worked h1 (or h2), so the pin catches that mistake."""
    l1, l2 = orollout.QuantLinear(W1, "mx"), orollout.QuantLinear(W2, "mx")
    g, rms = orollout.gelu, orollout.rmsnorm
    h = X.astype(np.float64)
    want1 = as_f64(vec(GOLD["block1"]["h"]))
    variants = {
        "no RMSNorm": h + l2(g(l1(h))),
        "RMSNorm after the first linear": h + l2(g(rms(l1(h)))),
        "GELU and RMSNorm exchanged": h + l2(rms(l1(g(h)))),
        "W1 and W2 exchanged": h + l1(g(l2(rms(h)))),
        "no residual": l2(g(l1(rms(h)))),
        "no GELU": h + l2(l1(rms(h))),
    }
    for name, v in variants.items():
        assert not np.array_equal(v[0], want1), name
    h1 = orollout.velocity(X, [l1], [l2])
    want2 = as_f64(vec(GOLD["block2"]["h"]))
    wrong_state = h1 + l2(g(l1(rms(h))))          # block 2 normalizes x instead of h1
    assert not np.array_equal(wrong_state[0], want2)
