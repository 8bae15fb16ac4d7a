"""MXFP4 block quantization -- oracle, test infrastructure only.

Format (one of the two fixed for the FP4 solver of the Sol-RL project page,
"Two-Stage Pipeline"; the pages themselves leave the layout open): blocks of
32 consecutive elements along the last axis K share one E8M0 scale, a pure
power of two 2^(S-127) stored as the byte S; each element is an E2M1 code.

Scale rule (reading, following the OCP Microscaling spec's conversion): with
amax the largest magnitude in the block, E = floor(log2(amax)) - 2 (2 is the
largest E2M1 exponent), clamped to [-127, 127]; an all-zero block takes the
clamped limit E = -127. The element codes are the nearest-even E2M1 codes of
x * 2^-E. A block whose amax / 2^E lies in (6, 8) saturates its largest
elements to 6 -- this is what the rule does, not a bug.
"""
import numpy as np

from . import e2m1

BLOCK = 32


def scale_exponent(amax):
    """E per block from exact floor(log2(amax)); frexp gives amax = m 2^e, m in [0.5, 1)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    E = e.astype(np.int64) - 1 - 2
    E = np.where(amax == 0, -127, E)
    return np.clip(E, -127, 127)


def quantize(x):
    """x: [rows, K] float array (fp32 or bf16 values, held exactly in float64).

    Returns (codes [rows, K/2] uint8, scales [rows, K/32] uint8)."""
    x = np.asarray(x, dtype=np.float64)
    rows, k = x.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32 for MXFP4")
    xb = x.reshape(rows, k // BLOCK, BLOCK)
    amax = np.abs(xb).max(axis=-1)
    E = scale_exponent(amax)
    y = np.ldexp(xb, -E[..., None])          # exact: a power-of-two rescale in float64
    nib = e2m1.encode(y).reshape(rows, k)
    return e2m1.pack(nib), (E + 127).astype(np.uint8)


def dequant(codes, scales):
    """Exact float64 values (-1)^s G[m] 2^(S-127)."""
    nib = e2m1.unpack(codes)
    rows, k = nib.shape
    vals = e2m1.decode(nib).reshape(rows, k // BLOCK, BLOCK)
    S = np.asarray(scales, dtype=np.int64)[:, : k // BLOCK]
    return np.ldexp(vals, (S - 127)[..., None]).reshape(rows, k)
