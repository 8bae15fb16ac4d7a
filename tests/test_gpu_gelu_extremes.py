"""The first linear's fused GELU + MXFP4 epilogues (fp4_gemm_panel_gelu_f32,
and fp4_gemm_panel_gelu for the bf16 reading) on hidden values built to
reach every case of their two passes.

The epilogue first runs a pass without branches: the table expansion for
every value (no evaluated erfc beyond |z| = 6) and the hardware converter
for every block. Where a wave's tile holds a block whose scale byte is below
103 or above 252 (all-tail or all-zero blocks, NaN from overflowing values),
it writes the tile again with the exact treatment. The outputs must be those
of the fp32 GEMM followed by the GELU quantizer (which treats every value
exactly), byte for byte, and the oracle's quantization of GELU of the exact
products outside the decision band.

Construction: B holds chosen values and A one or two unit entries per row,
so each hidden value is one chosen value or the sum of two. B's 32-blocks
along k are 32-row groups of the chosen matrix zt (B = zt^T), each group of
one column drawn as E2M1 grid values times one power of two, so B quantizes
exactly. Row groups and column ranges cover, per 128 x 128 wave tile:
  * ordinary values with z > 6 in every fourth column (first pass only; z > 6
    gives z);
  * whole blocks below -6 (the tile is redone);
  * blocks half below -6 down to -2^20, half ordinary (first pass only: the
    tail values give negative zero codes);
  * zero blocks and values near 7e18 (redone: scale byte 0, and NaN from the
    overflowing expansion);
  * rows that add two groups, giving sums within 0.012 of +-6 and mixtures
    of all of the above.
"""
import numpy as np
import pytest
import torch

from oracle import gemm as ogemm, rollout as orollout
from tests._parity import mx_codes_near_boundary_ok, panel_to_rows, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GRID = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
M, N, K = 512, 512, 256


def segment(rng, kind):
    """32 values of one (row group, column) segment, one power of two."""
    if kind == "zero":
        return np.zeros(32)
    if kind == "ord":
        t = int(rng.integers(-3, 1))
        return rng.choice(GRID, 32) * rng.choice([-1.0, 1.0], 32) * 2.0 ** t
    if kind == "neg":      # every value below -6
        t = int(rng.integers(2, 21))
        return -rng.choice(GRID[3:], 32) * 2.0 ** t
    if kind == "pos":      # every value above 6
        t = int(rng.integers(2, 6))
        return rng.choice(GRID[3:], 32) * 2.0 ** t
    if kind == "six":      # +-6 exactly
        return 6.0 * rng.choice([-1.0, 1.0], 32)
    if kind == "tiny":     # 2^-10 .. 0.012
        return rng.choice(GRID, 32) * rng.choice([-1.0, 1.0], 32) * 2.0 ** -9
    if kind == "huge":     # about 7e18 and beyond, both signs
        return rng.choice(GRID[4:], 32) * rng.choice([-1.0, 1.0], 32) * 2.0 ** 60
    raise ValueError(kind)


def chosen_values(seed):
    """zt [256, N]: kinds per (32-row group g, column n)."""
    rng = np.random.default_rng(seed)
    zt = np.empty((256, N))
    for g in range(8):
        for n in range(N):
            kind = "ord"
            if n < 128 and g < 4 and n % 4 == 0:
                kind = "pos"
            elif 128 <= n < 256 and g < 2:
                kind = "neg"
            elif n < 128 and g >= 4 and n % 2 == 0:
                kind = "neg"
            elif 128 <= n < 192 and g == 4:
                kind = "zero"
            elif 128 <= n < 256 and g == 5 and n % 16 == 8:
                kind = "huge"
            elif 256 <= n < 384 and g == 0:
                kind = "six"
            elif 256 <= n < 384 and g == 2:
                kind = "tiny"
            zt[32 * g:32 * g + 32, n] = segment(rng, kind)
    return zt


def operands():
    zt = chosen_values(7)
    b = np.zeros((N, K), np.float32)
    b[:, :256] = zt.T
    a = np.zeros((M, K), np.float32)
    for r in range(256):
        a[r, r] = 1.0
    for r in range(256, M):
        kk = r - 256
        a[r, kk] = 1.0
        a[r, (kk + 64) % 256] = 1.0
    return a, b


def test_fused_fp32_gelu_two_pass_cases(gpu_lib):
    a, b = operands()
    qa = gpu_lib.quantize(torch.from_numpy(a).to(DEV), "mx", layout="panel")
    qb = gpu_lib.quantize(torch.from_numpy(b).to(DEV), "mx", layout="panel")
    # B must hold the chosen values exactly
    bc, bs, _ = panel_to_rows(to_np(qb.codes), to_np(qb.scales), N, K)
    ac, as_, _ = panel_to_rows(to_np(qa.codes), to_np(qa.scales), M, K)
    c_exact, s_abs = ogemm.gemm_mx(ac, as_, bc, bs)
    np.testing.assert_array_equal(c_exact[:256], (a[:256].astype(np.float64) @ b.T.astype(np.float64)))

    z = gpu_lib.gemm(qa, qb, "f32", out=torch.empty((M, N), dtype=torch.float32, device=DEV))
    ref = gpu_lib.quantize(z, "mx", prologue="gelu", layout="panel")
    out = gpu_lib.gemm_gelu(qa, qb, exact=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(out.scales), to_np(ref.scales))
    np.testing.assert_array_equal(to_np(out.codes), to_np(ref.codes))

    zf = to_np(z).astype(np.float64)
    print(f"hidden values: {np.sum(zf < -6)} below -6, {np.sum(zf > 6)} above 6, "
          f"{np.sum(np.abs(np.abs(zf) - 6) < 0.0157)} within 0.0157 of +-6, {np.sum(zf == 0)} zero, "
          f"{np.sum(np.abs(zf) > 1e9)} beyond 1e9")
    assert np.sum(np.abs(np.abs(zf) - 6) < 0.0157) > 1000 and np.sum(np.abs(zf) > 1e9) > 100

    oc, osc, _ = panel_to_rows(to_np(out.codes), to_np(out.scales), M, N)
    bad, flips = mx_codes_near_boundary_ok(orollout.gelu(c_exact), oc, osc, band=1.13 * 1e-4 * s_abs)
    assert bad == 0, (bad, flips)


def test_fused_fp32_gelu_redo_leaves_other_tiles_alone(gpu_lib):
    """A single all-zero block in one wave tile makes only that tile take the
    second pass; the output equals the unfused pair either way, and a second
    call with the same inputs gives the same bytes."""
    rng = np.random.default_rng(3)
    a = (rng.choice(GRID, (M, K)) * rng.choice([-1.0, 1.0], (M, K)) * 0.25).astype(np.float32)
    b = (rng.choice(GRID, (N, K)) * rng.choice([-1.0, 1.0], (N, K)) * 0.125).astype(np.float32)
    a[130] = 0.0       # row 130: its blocks in every column tile are zero
    qa = gpu_lib.quantize(torch.from_numpy(a).to(DEV), "mx", layout="panel")
    qb = gpu_lib.quantize(torch.from_numpy(b).to(DEV), "mx", layout="panel")
    z = gpu_lib.gemm(qa, qb, "f32", out=torch.empty((M, N), dtype=torch.float32, device=DEV))
    ref = gpu_lib.quantize(z, "mx", prologue="gelu", layout="panel")
    out1 = gpu_lib.gemm_gelu(qa, qb, exact=True)
    out2 = gpu_lib.gemm_gelu(qa, qb, exact=True)
    torch.cuda.synchronize()
    for out in (out1, out2):
        np.testing.assert_array_equal(to_np(out.scales), to_np(ref.scales))
        np.testing.assert_array_equal(to_np(out.codes), to_np(ref.codes))


@pytest.mark.parametrize("which", ["extremes", "zero_row"])
def test_fused_bf16_gelu_two_pass_cases(gpu_lib, which):
    """fp4_gemm_panel_gelu (GELU of bf16(sum)) on the same operands: the
    first pass uses the hardware converter for every block, and a tile with
    a block whose scale byte is 2 or less (the zero blocks here) is written
    again with the ALU converter. Byte for byte the bf16 GEMM followed by the
    GELU quantizer."""
    if which == "extremes":
        a, b = operands()
    else:
        rng = np.random.default_rng(5)
        a = (rng.choice(GRID, (M, K)) * rng.choice([-1.0, 1.0], (M, K)) * 0.25).astype(np.float32)
        b = (rng.choice(GRID, (N, K)) * rng.choice([-1.0, 1.0], (N, K)) * 0.125).astype(np.float32)
        a[300] = 0.0
    qa = gpu_lib.quantize(torch.from_numpy(a).to(DEV), "mx", layout="panel")
    qb = gpu_lib.quantize(torch.from_numpy(b).to(DEV), "mx", layout="panel")
    z = gpu_lib.gemm(qa, qb, "bf16", out=torch.empty((M, N), dtype=torch.bfloat16, device=DEV))
    ref = gpu_lib.quantize(z, "mx", prologue="gelu", layout="panel")
    out = gpu_lib.gemm_gelu(qa, qb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(out.scales), to_np(ref.scales))
    np.testing.assert_array_equal(to_np(out.codes), to_np(ref.codes))
    assert (to_np(ref.scales) <= 2).any()      # the second pass was needed somewhere
