"""E2M1 (FP4) element code -- oracle, test infrastructure only.

An E2M1 value has 1 sign bit, 2 exponent bits and 1 mantissa bit; its
non-negative magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}. The pages name the
4-bit float format (Sol-RL project page, "Two-Stage Pipeline", NVFP4 solver)
without defining rounding; the reading used here is the plain one for an IEEE-
like format: round to the nearest representable magnitude, ties to the even
code (the one whose mantissa bit is 0), saturate beyond 6, and keep the sign
(so -0.0 and negatives that round to zero get the sign bit).

Nibble = (sign << 3) | magnitude index. Two nibbles pack into one byte, the
element with the even index in the low nibble.
"""
import numpy as np

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def encode(v):
    """Nearest-even E2M1 nibble of each real value in `v` (float64 array).

    Distances to the 8 magnitudes are exact in float64 while |v| < 8; any
    magnitude from 6 up has 6 as its nearest point (saturation), which is
    taken directly because rounded distances of huge values all tie.
    """
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8)
    a = np.abs(v)
    dist = np.abs(a[..., None] - GRID)                  # [..., 8]
    dmin = dist.min(axis=-1, keepdims=True)
    at_min = dist == dmin
    even = (np.arange(8) % 2) == 0
    # two candidates only at an exact midpoint; exactly one of them is even
    two = at_min.sum(axis=-1) == 2
    pick_even = np.argmax(at_min & even, axis=-1)
    pick_any = np.argmax(at_min, axis=-1)
    idx = np.where(two, pick_even, pick_any)
    idx = np.where(a >= 6.0, 7, idx).astype(np.uint8)
    return (sign << 3) | idx


def decode(nib):
    nib = np.asarray(nib, dtype=np.uint8)
    mag = GRID[nib & 7]
    return np.where(nib & 8, -mag, mag)


def pack(nib):
    """[..., K] nibbles -> [..., K/2] bytes, element 2j in the low nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    assert nib.shape[-1] % 2 == 0
    lo = nib[..., 0::2] & 0xF
    hi = nib[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out
