"""Pins for the oracle's E2M1 element code (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import e2m1

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def grid_from_bits():
    """E2M1 magnitudes from the bit fields: e (2 bits, bias 1), m (1 bit)."""
    vals = []
    for code in range(8):
        e, m = code >> 1, code & 1
        vals.append(m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))
    return vals


def threshold_code(a):
    """Magnitude index by the explicit decision thresholds (ties resolved to
    the even index): <=.25:0 <.75:1 <=1.25:2 <1.75:3 <=2.5:4 <3.5:5 <=5:6 else 7."""
    if a <= 0.25:
        return 0
    if a < 0.75:
        return 1
    if a <= 1.25:
        return 2
    if a < 1.75:
        return 3
    if a <= 2.5:
        return 4
    if a < 3.5:
        return 5
    if a <= 5.0:
        return 6
    return 7


def test_grid_matches_bit_fields():
    assert list(e2m1.GRID) == grid_from_bits()


def test_hand_grid_and_midpoints():
    g = load("e2m1_grid.json")
    for key in ("grid", "midpoints", "saturating"):
        for v, idx in g[key]:
            assert e2m1.encode(np.array([v]))[0] == idx, (key, v)
            assert e2m1.encode(np.array([-v]))[0] == idx | 8, (key, -v)


def test_signed_zero():
    assert e2m1.encode(np.array([0.0]))[0] == 0
    assert e2m1.encode(np.array([-0.0]))[0] == 8
    assert e2m1.encode(np.array([-0.1]))[0] == 8      # rounds to zero, keeps sign
    assert e2m1.encode(np.array([-0.25]))[0] == 8     # tie to even (zero)


def test_threshold_form_dense_sweep():
    """Every fp32 value near each threshold, plus a regular sweep of [0, 10]."""
    thr = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = [np.float32(v) for v in np.linspace(0, 10, 20001)]
    for t in thr:
        x = np.float32(t)
        lo = hi = x
        for _ in range(6):
            lo = np.nextafter(lo, np.float32(0))
            hi = np.nextafter(hi, np.float32(100))
            vals += [lo, hi]
        vals.append(x)
    v = np.array(vals, dtype=np.float32).astype(np.float64)
    got = e2m1.encode(v)
    want = np.array([threshold_code(a) for a in v], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_bruteforce_nearest_16_codes():
    """Against a brute-force search over all 16 signed codes, with the
    tie-break to the even mantissa bit (bit 0)."""
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.uniform(-8, 8, 4000), np.arange(-7, 7.01, 0.25)])
    signed = [(c, (-1 if c & 8 else 1) * grid_from_bits()[c & 7]) for c in range(16)]
    got = e2m1.encode(v)
    for x, q in zip(v, got):
        best = None
        for c, val in signed:
            if (c & 8) != (8 if np.signbit(x) else 0):
                continue      # the sign is kept, so only same-signed codes compete
            d = abs(x - val)
            key = (d, c & 1)
            if best is None or key < best[0]:
                best = (key, c)
        assert q == best[1], (x, q, best)


def test_pack_unpack_low_nibble_first():
    nib = np.array([[1, 9, 3, 5]], dtype=np.uint8)
    packed = e2m1.pack(nib)
    assert packed.tolist() == [[0x91, 0x53]]
    np.testing.assert_array_equal(e2m1.unpack(packed), nib)


def test_encode_is_monotone_in_magnitude():
    """For a fixed sign the magnitude index never decreases as |x| grows
    (the property the exhaustive GPU sweeps rely on to check whole runs of
    patterns from their ends): every fp32 pattern within 2^14 ulps of each
    decision point and of each grid value, plus a stride through all finite
    patterns, in increasing order."""
    pts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 8.0]
    parts = [np.arange(0, 0x7F800000, 4099, dtype=np.int64)]
    for v in pts:
        b = int(np.array(v, np.float32).view(np.uint32))
        parts.append(np.arange(b - (1 << 14), b + (1 << 14), dtype=np.int64))
    p = np.unique(np.concatenate(parts)).astype(np.uint32)
    x = p.view(np.float32).astype(np.float64)
    for sign in (1.0, -1.0):
        nib = e2m1.encode(sign * x)
        assert np.all(np.diff((nib & 7).astype(np.int64)) >= 0)
        assert np.all((nib >> 3) == (1 if sign < 0 else 0))
