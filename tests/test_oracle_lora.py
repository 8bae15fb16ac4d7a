"""Pins of the LoRA-merge oracle against values fixed by the definition
W' = W + s (B A), not by re-calling its matmul:

  * exact rational arithmetic (fractions.Fraction) with explicit loops on
    small non-square shapes, where a transposed operand, a dropped term, a
    wrong sign or a scale applied to W would all show;
  * closed forms: all-ones adapters give W + s r; a rank-one adapter gives
    W + s b_n a_k element by element;
  * the identity cases s = 0 and B = 0, which must return W exactly;
  * the quantized merge of an adapter that cancels W exactly gives the
    all-zero blocks (scale byte 0, codes 0).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import lora, mxfp4


def exact_merge(w, b, a, s):
    n, k = w.shape
    r = b.shape[1]
    out = [[None] * k for _ in range(n)]
    for i in range(n):
        for j in range(k):
            acc = Fraction(0)
            for t in range(r):
                acc += Fraction(float(b[i, t])) * Fraction(float(a[t, j]))
            out[i][j] = Fraction(float(w[i, j])) + Fraction(float(s)) * acc
    return out


@pytest.mark.parametrize("n,k,r,seed", [(3, 32, 2, 0), (5, 7, 4, 1), (1, 64, 1, 2), (4, 3, 6, 3)])
def test_merge_against_exact_rationals(n, k, r, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k)).astype(np.float32)
    b = rng.standard_normal((n, r)).astype(np.float32)
    a = rng.standard_normal((r, k)).astype(np.float32)
    s = np.float32(0.37)
    got = lora.merge(w, b, a, s)
    ref = exact_merge(w, b, a, s)
    for i in range(n):
        for j in range(k):
            x = ref[i][j]
            # float64 evaluation error: at most ~ (r + 2) 2^-53 of the magnitudes involved
            mag = abs(float(w[i, j])) + abs(float(s)) * sum(abs(float(b[i, t]) * float(a[t, j])) for t in range(r))
            assert abs(Fraction(float(got[i, j])) - x) <= Fraction((r + 2) * 2.0 ** -53 * mag)


def test_all_ones_adapter_closed_form():
    w = np.arange(12, dtype=np.float32).reshape(3, 4) - 5.0
    r, s = 8, 0.25
    got = lora.merge(w, np.ones((3, r), np.float32), np.ones((r, 4), np.float32), s)
    np.testing.assert_array_equal(got, w.astype(np.float64) + s * r)


def test_rank_one_outer_product():
    w = np.array([[1.0, -2.0, 0.5], [0.0, 4.0, -1.5]], np.float32)
    b = np.array([[2.0], [-3.0]], np.float32)
    a = np.array([[0.5, 1.0, -4.0]], np.float32)
    s = 0.5
    want = np.array([[1.0 + 0.5 * 2.0 * 0.5, -2.0 + 0.5 * 2.0 * 1.0, 0.5 + 0.5 * 2.0 * -4.0],
                     [0.0 + 0.5 * -3.0 * 0.5, 4.0 + 0.5 * -3.0 * 1.0, -1.5 + 0.5 * -3.0 * -4.0]])
    np.testing.assert_array_equal(lora.merge(w, b, a, s), want)


def test_identity_cases():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((6, 32)).astype(np.float32)
    b = rng.standard_normal((6, 4)).astype(np.float32)
    a = rng.standard_normal((4, 32)).astype(np.float32)
    np.testing.assert_array_equal(lora.merge(w, b, a, 0.0), w)
    np.testing.assert_array_equal(lora.merge(w, np.zeros_like(b), a, 3.0), w)


def test_cancelling_adapter_quantizes_to_zero_blocks():
    # W = -s B A exactly (small integers): the merged weight is all zeros
    b = np.array([[1.0, 2.0], [3.0, -1.0]], np.float32)
    a = np.tile(np.array([[1.0], [2.0]], np.float32), (1, 32))
    s = 0.5
    w = (-s * (b.astype(np.float64) @ a)).astype(np.float32)
    merged = lora.merge(w, b, a, s)
    assert not merged.any()
    codes, scales = mxfp4.quantize(merged)
    assert not codes.any() and not scales.any()


def test_shape_errors():
    w = np.zeros((3, 32), np.float32)
    with pytest.raises(ValueError):
        lora.merge(w, np.zeros((3, 2)), np.zeros((3, 32)), 1.0)
    with pytest.raises(ValueError):
        lora.merge(w, np.zeros((2, 2)), np.zeros((2, 32)), 1.0)
