"""Pins for the oracle's NVFP4-style quantizer (CPU only)."""
import json
import os

import numpy as np
import torch

from oracle import e2m1, nvfp4

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_blocks():
    with open(os.path.join(GOLD, "nv_blocks.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        nb = len(case["blocks"])
        x = np.zeros((1, 16 * nb), dtype=np.float32)
        for b, vals in enumerate(case["blocks"]):
            x[0, 16 * b: 16 * b + len(vals)] = np.array(vals, dtype=np.float32)
        codes, scales, sg = nvfp4.quantize(x)
        assert abs(float(sg) - case["s_g"]) <= 1e-12, case["name"]
        assert scales[0].tolist() == case["scales"], case["name"]
        nib = e2m1.unpack(codes)[0]
        for b, want in enumerate(case["nibbles"]):
            assert nib[16 * b: 16 * b + len(want)].tolist() == want, case["name"]


def test_e4m3_encode_matches_torch_cast():
    """torch's float8_e4m3fn cast rounds to nearest even; compare on [0, 448]."""
    rng = np.random.default_rng(5)
    s = np.concatenate([
        rng.uniform(0, 448, 20000), np.exp2(rng.uniform(-12, 8.8, 20000)),
        nvfp4.e4m3_values(),                               # exact codes
        (nvfp4.e4m3_values()[:-1] + nvfp4.e4m3_values()[1:]) / 2,   # exact ties
    ]).astype(np.float32)
    s = s[s <= 448]
    want = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = nvfp4.e4m3_encode(s.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_e4m3_values_from_bit_fields_and_saturation():
    v = nvfp4.e4m3_values()
    assert v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9
    assert np.all(np.diff(v) > 0)
    assert nvfp4.e4m3_encode(np.array([463.9, 470.0, 1e9])).tolist() == [0x7E] * 3
    # far above 448, where s - 448 rounds back to s in float64, and +inf
    # (a block amax over a tiny given tensor scale): still the largest code
    assert nvfp4.e4m3_encode(np.array([1e20, 5e21, 3e38, np.inf])).tolist() == [0x7E] * 4
    assert nvfp4.e4m3_encode(np.array([2.0 ** -10])).tolist() == [0]       # tie to even zero
    assert nvfp4.e4m3_encode(np.array([1.5 * 2.0 ** -9])).tolist() == [2]  # tie to even code 2


def test_sign_symmetry_and_block_max_saturates_to_448():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    c1, s1, g1 = nvfp4.quantize(x)
    c2, s2, g2 = nvfp4.quantize(-x)
    np.testing.assert_array_equal(c2, c1 ^ 0x88)
    np.testing.assert_array_equal(s1, s2)
    assert g1 == g2
    # the block holding the tensor amax gets scale 448 (0x7E)
    r, col = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert s1[r, col // 16] == 0x7E


def test_codes_are_nearest_given_scale():
    """Every code is the nearest-even E2M1 point to fl32(x/d) -- brute force
    over the 8 magnitudes, independent of the oracle's encode."""
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((4, 64)) * 3).astype(np.float32)
    codes, scales, sg = nvfp4.quantize(x)
    nib = e2m1.unpack(codes)
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for r in range(4):
        for k in range(64):
            d = np.float32(np.float32(nvfp4.e4m3_decode(scales[r, k // 16])) * sg)
            y = float(np.float32(x[r, k] / d))
            best = min(range(8), key=lambda i: (abs(abs(y) - grid[i]), i & 1))
            assert nib[r, k] & 7 == best and (nib[r, k] >> 3) == int(np.signbit(x[r, k]))


def test_round_trip_error_bound():
    """|x - dequant| <= half a grid step times the block scale, for blocks
    that do not saturate (max step 2 near 6 -> bound 1 * scale)."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((32, 128)).astype(np.float32)
    codes, scales, sg = nvfp4.quantize(x)
    xd = nvfp4.dequant(codes, scales, sg)
    bs = np.repeat(nvfp4.e4m3_decode(scales) * float(sg), 16, axis=1)
    assert np.all(np.abs(x - xd) <= 1.0 * bs * (1 + 1e-6))


def test_zero_tensor_and_given_scale():
    c, s, g = nvfp4.quantize(np.zeros((2, 32), dtype=np.float32))
    assert g == 1.0 and not c.any() and not s.any()
    x = np.ones((1, 16), dtype=np.float32)
    c, s, g = nvfp4.quantize(x, s_g=np.float32(1.0))
    # s_f = 1/6 -> E4M3 nearest to 0.1667 is 0.171875 (code 0x2B)... d = 0.171875, 1/d = 5.818 -> 6
    assert g == 1.0 and s[0, 0] == nvfp4.e4m3_encode(np.array([np.float32(1) / np.float32(6)]))[0]
    assert e2m1.unpack(c)[0, 0] == 7
