"""NVFP4-style block quantization -- oracle, test infrastructure only.

The pages name NVFP4 as the rollout format (Sol-RL project page, "Two-Stage
Pipeline"; aitrends summary, Stage-1 paragraph: weights quantized to NVFP4)
but never define it. The variant fixed here: blocks of 16 along K, each with
an E4M3 (OCP E4M3FN: bias 7, max 448, subnormals to 2^-9) scale, plus one fp32
scale for the whole tensor, applied per block.

Steps, all IEEE fp32 and correctly rounded, in this order (no fused
multiply-add):
  1. A_t = max |x| over the whole [rows, K] argument; s_g = A_t / 2688
     (2688 = 6 * 448), or 1 when that quotient is 0 (an all-zero tensor, or
     one so small that the quotient underflows -- every code is then a signed
     zero either way); or s_g supplied by the caller.
  2. per block: a_b = block amax; tau = 6 * s_g; s_f = a_b / tau.
  3. S = E4M3 code of s_f, round to nearest even, saturating at 448.
  4. d = dec(S) * s_g. If d == 0 the block's codes are signed zeros; otherwise
     each code is the nearest-even E2M1 code of x / d.
Dequantized value = (-1)^s G[m] dec(S) s_g, exact in float64.
"""
import numpy as np

from . import e2m1

BLOCK = 16
F32 = np.float32


def e4m3_values():
    """Exact values of the 127 finite non-negative E4M3FN codes 0x00..0x7E."""
    vals = np.empty(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3_values()


def e4m3_decode(code):
    return _E4M3[np.asarray(code, dtype=np.int64)]


def e4m3_encode(s):
    """Nearest finite E4M3 code of non-negative s, ties to the even code.

    Picking the nearest of the finite codes saturates at 448 (the IEEE rule
    would overflow only at >= 464, and there is no code above 448). s is
    clamped to 448 first: for s far above it (or infinite) the distances
    s - value all round to the same float64, and the nearest would be lost."""
    s = np.minimum(np.asarray(s, dtype=np.float64), 448.0)
    dist = np.abs(s[..., None] - _E4M3)
    dmin = dist.min(axis=-1, keepdims=True)
    at_min = dist == dmin
    even = (np.arange(127) % 2) == 0
    two = at_min.sum(axis=-1) == 2
    return np.where(two, np.argmax(at_min & even, axis=-1),
                    np.argmax(at_min, axis=-1)).astype(np.uint8)


def tensor_scale(x):
    """Step 1: s_g = fl32(A_t / 2688); 1 where that is 0."""
    at = F32(np.abs(np.asarray(x, dtype=F32)).max()) if np.size(x) else F32(0)
    sg = F32(at / F32(2688.0))
    return F32(1.0) if sg == 0 else sg


def quantize(x, s_g=None):
    """x: [rows, K] (fp32 or bf16 values). Returns (codes [rows,K/2], scales
    [rows,K/16] uint8 E4M3, s_g float32)."""
    x = np.asarray(x, dtype=F32)
    rows, k = x.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 16 for NVFP4")
    sg = tensor_scale(x) if s_g is None else F32(s_g)
    xb = x.reshape(rows, k // BLOCK, BLOCK)
    ab = np.abs(xb).max(axis=-1)                       # exact in fp32
    tau = F32(F32(6.0) * sg)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        sf = (ab / tau).astype(F32)                    # fp32 division, correctly rounded
    S = e4m3_encode(sf.astype(np.float64))
    d = (e4m3_decode(S).astype(F32) * sg).astype(F32)  # exact decode, one fp32 multiply
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = (xb / d[..., None]).astype(F32)
    nib = e2m1.encode(y.astype(np.float64))
    zero_blk = (d == 0)[..., None]
    nib = np.where(zero_blk, (np.signbit(xb).astype(np.uint8) << 3), nib)
    return e2m1.pack(nib.reshape(rows, k).astype(np.uint8)), S, sg


def dequant_unscaled(codes, scales):
    """G[m] dec(S) per element (no tensor scale), exact in float64."""
    nib = e2m1.unpack(codes)
    rows, k = nib.shape
    vals = e2m1.decode(nib).reshape(rows, k // BLOCK, BLOCK)
    sc = e4m3_decode(np.asarray(scales)[:, : k // BLOCK])
    return (vals * sc[..., None]).reshape(rows, k)


def dequant(codes, scales, s_g):
    return dequant_unscaled(codes, scales) * np.float64(F32(s_g))
