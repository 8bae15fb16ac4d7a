"""Exhaustive element-rounding sweeps of the quantizers' FP4 conversion
against the oracle, over every fp32 bit pattern of a range, both signs.

The MXFP4 quantizer converts through gfx950's scaled FP4 convert (blocks
with S >= 3) or an exact ALU path (S <= 2); the NVFP4-style quantizer feeds
its correctly rounded quotients to the same convert with scale 1. Each case
builds blocks whose first element pins the block scale and whose other
elements walk consecutive fp32 bit patterns:
  * MX, S = 127 (scale 2^0): every |x| < 8 -- every input the element rule
    can see at that scale, subnormals, -0 and the saturation range included;
  * MX, S = 252 (the largest scale an fp32 block can take): every finite x;
  * MX, S = 0..3: every |x| < 8 * 2^(S - 127), where fp32 subnormal elements
    round to non-zero codes (S = 1, 2) or to signed zeros (S = 3);
  * NVFP4-style with a given tensor scale 2^-8 and block amax 6, so that
    the block's E4M3 scale is 256 and its divisor d = 1: every |x| <= 6.375
    (the largest block amax that keeps d = 1).

The comparison is complete without evaluating the oracle 6.5e9 times: for a
fixed sign the oracle's magnitude code is a non-decreasing function of |x|
(nearest-point rounding on a sorted grid, ties to the even neighbour,
saturation above 6; pinned on the CPU in test_oracle_e2m1), and positive
fp32 bit patterns are sorted like their values. The GPU's codes over the
sweep are split into maximal runs of one code (on the GPU); the oracle is
evaluated at both ends of every run. Where it gives the run's code at both
ends it gives it at every pattern in between, so every element is checked.
A random sample of whole rows is also compared element by element.
"""
import numpy as np
import pytest
import torch

from oracle import e2m1, mxfp4, nvfp4
from tests._parity import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F32_INF_BITS = 0x7F800000


def f32_bits(v):
    return int(np.array(v, np.float32).view(np.uint32))


def patterns_to_f32(p, sign):
    """uint32 patterns (host int array) with the sign bit set or not -> float32."""
    p = np.asarray(p, dtype=np.uint64) | (np.uint64(0x80000000) if sign else np.uint64(0))
    return p.astype(np.uint32).view(np.float32)


def gpu_patterns(start, count_rows, per_row, hi, sign):
    """float32 [count_rows, per_row] of consecutive bit patterns start.. (the
    tail past hi repeats the last pattern), on the GPU."""
    p = torch.arange(start, start + count_rows * per_row, device=DEV, dtype=torch.int64).clamp_(max=hi - 1)
    if sign:
        p -= 1 << 31  # p | 0x80000000 as a two's-complement int32
    return p.to(torch.int32).view(torch.float32).view(count_rows, per_row)


def runs_of(nib, count):
    """(first index, last index, code) of each maximal run of equal codes in
    nib[:count] (a uint8 GPU vector), as host arrays."""
    nib = nib[:count]
    ch = torch.nonzero(nib[1:] != nib[:-1]).flatten() + 1
    first = torch.cat([torch.zeros(1, dtype=ch.dtype, device=DEV), ch])
    last = torch.cat([ch - 1, torch.full((1,), count - 1, dtype=ch.dtype, device=DEV)])
    return to_np(first).astype(np.int64), to_np(last).astype(np.int64), to_np(nib[first]).astype(np.uint8)


def unpack_gpu(codes):
    """[rows, k/2] uint8 GPU codes -> [rows, k] nibbles (element 2j low)."""
    return torch.stack([codes & 0xF, codes >> 4], dim=-1).reshape(codes.shape[0], -1)


def sweep(case, quantize_gpu, oracle_codes, pin, block, hi, sign, expect_scale, rows_per_chunk=1 << 21, seed=0):
    """Run one sweep; returns the number of patterns checked. quantize_gpu:
    fp32 [rows, block] GPU tensor -> (nibbles [rows, block] GPU, scale bytes
    [rows] GPU); oracle_codes: fp32 [rows, block] host array -> (nibbles,
    scale bytes) from the oracle."""
    per_row = block - 1
    rng = np.random.default_rng(seed)
    firsts, lasts, codes = [], [], []
    sample_x, sample_nib = [], []
    checked = 0
    for start in range(0, hi, rows_per_chunk * per_row):
        count = min(hi - start, rows_per_chunk * per_row)
        rows = -(-count // per_row)
        x = torch.empty(rows, block, dtype=torch.float32, device=DEV)
        x[:, 0] = float(pin)
        x[:, 1:] = gpu_patterns(start, rows, per_row, hi, sign)
        nib, sc = quantize_gpu(x)
        bad_scale = int((sc != expect_scale).sum())
        assert bad_scale == 0, f"{case}: {bad_scale} block scales differ from {expect_scale} (chunk at {start:#x})"
        f, l, c = runs_of(nib[:, 1:].reshape(-1), count)
        firsts.append(f + start)
        lasts.append(l + start)
        codes.append(c)
        pick = torch.from_numpy(rng.choice(rows, size=min(rows, 64), replace=False)).to(DEV)
        sample_x.append(to_np(x[pick]))
        sample_nib.append(to_np(nib[pick]))
        checked += count
    first, last, code = np.concatenate(firsts), np.concatenate(lasts), np.concatenate(codes)
    # the oracle at both ends of every run
    ends = np.concatenate([first, last])
    want = np.concatenate([code, code])
    xb = np.zeros((len(ends), block), np.float32)
    xb[:, 0] = pin
    xb[:, 1] = patterns_to_f32(ends, sign)
    on, osc = oracle_codes(xb)
    assert (osc == expect_scale).all(), f"{case}: the oracle's scale differs from the pinned one"
    bad = np.nonzero(on[:, 1] != want)[0]
    if len(bad):
        i = bad[0]
        v = xb[i, 1]
        raise AssertionError(f"{case}: x = {v!r} ({int(ends[i]):#010x}, sign {sign}): GPU code {want[i]:#x}, "
                             f"oracle {on[i, 1]:#x}; {len(bad)} of {len(ends)} run ends differ")
    # a random sample of whole rows, element by element
    sx, sn = np.concatenate(sample_x), np.concatenate(sample_nib)
    on, _ = oracle_codes(sx)
    np.testing.assert_array_equal(sn, on, err_msg=f"{case}: sampled rows differ")
    print(f"{case} sign {int(sign)}: {checked} patterns, {len(first)} runs")
    return checked


def mx_gpu(x):
    import fp4_quantized_diffusion_amd as fq
    q = fq.quantize(x, "mx")
    return unpack_gpu(q.codes[:, : x.shape[1] // 2]), q.scales[:, 0]


def mx_oracle(x):
    c, s = mxfp4.quantize(x)
    return e2m1.unpack(c), s[:, 0]


@pytest.mark.parametrize("S", [127, 252, 0, 1, 2, 3])
@pytest.mark.parametrize("sign", [False, True])
def test_mx_element_rounding_exhaustive(gpu_lib, S, sign):
    """Every fp32 pattern below 8 * 2^(S - 127) in magnitude (every finite
    value for S = 252) in blocks whose pin fixes scale byte S."""
    E = S - 127
    if S == 0:  # every block amax below 2^-124 gives S = 0: no pin needed
        pin, hi = np.float32(0.0), f32_bits(np.ldexp(1.0, -124))
    else:
        pin = np.float32(np.ldexp(4.0, E))
        hi = F32_INF_BITS if S == 252 else f32_bits(np.ldexp(8.0, E))
    n = sweep(f"MX S={S}", mx_gpu, mx_oracle, pin, 32, hi, sign, S)
    assert n == hi


def nv_gpu(x):
    import fp4_quantized_diffusion_amd as fq
    q = fq.quantize(x, "nv", tensor_scale=torch.full((1,), 2.0 ** -8, dtype=torch.float32, device=DEV))
    return unpack_gpu(q.codes[:, : x.shape[1] // 2]), q.scales[:, 0]


def nv_oracle(x):
    c, s, _ = nvfp4.quantize(x, s_g=np.float32(2.0 ** -8))
    return e2m1.unpack(c), s[:, 0]


@pytest.mark.parametrize("sign", [False, True])
def test_nv_element_rounding_exhaustive(gpu_lib, sign):
    """NVFP4-style blocks of 16 with tensor scale 2^-8 and a pinned amax of 6:
    s_f = 6 / fl(6 * 2^-8) = 256, its E4M3 code 0x78 and d = 1, so the
    quotient is x itself and the conversion sees every pattern |x| <= 6.375
    (amax up to 6.375 keeps s_f <= 272, which rounds to 256)."""
    hi = f32_bits(6.375) + 1
    expect = int(nv_oracle(np.full((1, 16), 6.0, np.float32))[1][0])
    assert expect == 0x78
    n = sweep("NV d=1", nv_gpu, nv_oracle, np.float32(6.0), 16, hi, sign, expect, rows_per_chunk=1 << 22)
    assert n == hi
