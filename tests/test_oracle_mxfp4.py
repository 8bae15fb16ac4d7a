"""Pins for the oracle's MXFP4 block quantizer (CPU only)."""
import json
import os

import numpy as np

from oracle import e2m1, mxfp4

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def block_from(values, n=32):
    x = np.zeros((1, n), dtype=np.float32)
    for i, v in enumerate(values):
        x[0, i] = np.float32(float(v))
    return x


def test_hand_worked_blocks():
    with open(os.path.join(GOLD, "mx_blocks.json")) as f:
        g = json.load(f)
    for b in g["blocks"]:
        x = block_from(b["x"])
        codes, scales = mxfp4.quantize(x)
        assert scales[0, 0] == b["scale"], b["name"]
        nib = e2m1.unpack(codes)[0]
        if "bytes" in b:
            assert codes[0].tolist() == b["bytes"], b["name"]
        if "nibbles" in b:
            k = len(b["nibbles"])
            assert nib[:k].tolist() == b["nibbles"], b["name"]
            assert not nib[k:].any(), b["name"]
        if "dequant" in b:
            d = mxfp4.dequant(codes, scales)[0]
            np.testing.assert_array_equal(d[: len(b["dequant"])], b["dequant"])


def random_representable(rng, rows, blocks):
    """Blocks of grid values times 2^e (one e per block, in range), at least
    one non-zero element per block."""
    nib = rng.integers(0, 16, size=(rows, blocks, 32)).astype(np.uint8)
    nib[..., 0] = rng.integers(1, 8, size=(rows, blocks)) | (rng.integers(0, 2, size=(rows, blocks)) << 3)
    e = rng.integers(-100, 100, size=(rows, blocks))
    v = np.ldexp(e2m1.decode(nib), e[..., None])
    return v.reshape(rows, blocks * 32).astype(np.float32)


def test_round_trip_of_representable_blocks():
    rng = np.random.default_rng(1)
    x = random_representable(rng, 64, 8)
    codes, scales = mxfp4.quantize(x)
    np.testing.assert_array_equal(mxfp4.dequant(codes, scales), x.astype(np.float64))


def test_idempotence():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    c1, s1 = mxfp4.quantize(x)
    c2, s2 = mxfp4.quantize(mxfp4.dequant(c1, s1).astype(np.float32))
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)


def test_sign_symmetry():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    x[0, :5] = 0.0
    c1, s1 = mxfp4.quantize(x)
    c2, s2 = mxfp4.quantize(-x)
    np.testing.assert_array_equal(c2, c1 ^ 0x88)
    np.testing.assert_array_equal(s1, s2)


def test_power_of_two_scaling():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    c0, s0 = mxfp4.quantize(x)
    for j in (-30, -1, 1, 7, 40):
        cj, sj = mxfp4.quantize(np.ldexp(x, j).astype(np.float32))
        np.testing.assert_array_equal(cj, c0)
        np.testing.assert_array_equal(sj.astype(int), s0.astype(int) + j)


def test_scale_is_floor_log2_minus_two():
    """amax in [2^p, 2^(p+1)) gives S = p - 2 + 127 -- checked at both ends of
    each binade with math.frexp-free integer reasoning."""
    for p in range(-120, 120, 7):
        for a in (2.0 ** p, np.nextafter(np.float32(2.0 ** (p + 1)), np.float32(0))):
            x = block_from([a])
            _, s = mxfp4.quantize(x)
            assert int(s[0, 0]) == p - 2 + 127, (p, a)


def test_subnormal_and_tiny_blocks_clamp():
    x = block_from([1e-40, -3e-41])             # fp32 subnormals
    c, s = mxfp4.quantize(x)
    assert s[0, 0] == 0
    # 1e-40 * 2^127 = 1.70e-2 -> 0 ; the sign of -3e-41 is kept
    nib = e2m1.unpack(c)[0]
    assert nib[0] == 0 and nib[1] == 8
    x = block_from([2.0 ** -125])               # E = -127 exactly: 2^-125 * 2^127 = 4
    c, s = mxfp4.quantize(x)
    assert s[0, 0] == 0 and e2m1.unpack(c)[0][0] == 6


def test_largest_finite_input():
    x = block_from([np.finfo(np.float32).max, -1.0])
    c, s = mxfp4.quantize(x)
    assert s[0, 0] == 127 + 127 - 2
    assert e2m1.unpack(c)[0][0] == 7


def test_saturation_band():
    """amax / 2^E in (6, 8): the block maximum saturates to 6 * 2^E."""
    x = block_from([7.0, 3.0])
    c, s = mxfp4.quantize(x)
    assert s[0, 0] == 127
    np.testing.assert_array_equal(mxfp4.dequant(c, s)[0, :2], [6.0, 3.0])
