"""The argument behind the fused fp32 GELU epilogue's first pass, checked on
the CPU in a float32 emulation of its arithmetic (the kernel itself is
checked on the GPU by tests/test_gpu_gelu_extremes.py).

The first pass evaluates the table expansion for every value, with no
evaluated erfc beyond |z| = 6, and the table's entries above 6 are zero. The
pass keeps the exact treatment's codes wherever every block's scale byte is
at least 103 and at most 252, because beyond |z| = 6 the expansion gives:
  * z itself for z > 6 (as the evaluated erfc does);
  * a negative value below 6e-9 in magnitude, or -0, for z < -6 (where the
    evaluated erfc gives a negative value below 6e-9 or -0: |z| Q(|z|) is at
    most 6 Q(6) = 5.92e-9 there);
  * NaN once the expansion overflows (and for NaN or infinite z),
which make a block's scale byte 253.

The emulation rounds every operation to float32 (fma through a float64
product and sum, then one rounding: exact for the products, and the sums
here are far from float32 ties). Table entries come from float64 erfc and
exp; the kernel's own entries differ from them by a few ulps, far inside the
margins below."""
import math

import numpy as np

F = np.float32


def fma(a, b, c):
    return F(np.float64(a) * np.float64(b) + np.float64(c))


def bf16_rne(x):
    u = np.array([x], np.float32).view(np.uint32)[0]
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return np.array([r], np.uint32).view(np.float32)[0]


LO, HI, TAYLOR_MAX = F(2.0 ** -10), F(16.0), 6.0


def entry(ac):
    if ac > TAYLOR_MAX:
        return F(0), F(0)
    a = float(ac)
    return F(0.5 * math.erfc(a / math.sqrt(2))), F(math.exp(-a * a / 2) / math.sqrt(2 * math.pi))


def first_pass_gelu(z):
    """The first pass's value for one fp32 z: the table entry at the bf16
    rounding of |z| (clamped to [2^-10, 16]) and the fourth-order expansion
    in x = a_c d, then z Phi(z) = fma(-|z|, Q, max(z, -0))."""
    z = F(z)
    ac = bf16_rne(abs(z))
    ac = min(max(ac, LO), HI) if ac == ac else HI
    q0, phi = entry(ac)
    with np.errstate(over="ignore", invalid="ignore"):
        d = F(abs(z) - ac)
        x = F(ac * d)
        b = fma(fma(fma(x, F(-1 / 24), F(1 / 6)), x, F(-0.5)), x, F(1))
        b = fma(F(d * d), fma(x, F(0.125), F(-1 / 6)), b)
        q = fma(-phi, F(b * d), q0)
        return fma(-abs(z), q, max(z, F(-0.0)) if z != 0 else z)


def grid():
    rng = np.random.default_rng(0)
    lin = np.linspace(6.0, 17.0, 20001)
    log = np.exp(rng.uniform(math.log(6.0), math.log(1e12), 20000))
    z = np.concatenate([lin, log, [np.nextafter(F(6), F(7)), 6.0078125, 6.015625, 6.0234375, 16.0, 16.03125]])
    return z.astype(np.float32)[z.astype(np.float32) > F(6)]


def test_positive_tail_gives_z_or_nan():
    for z in grid():
        g = first_pass_gelu(z)
        assert g == z or math.isnan(g), (z, g)


def test_negative_tail_is_a_tiny_negative_or_nan():
    worst = 0.0
    for z in grid():
        g = first_pass_gelu(-z)
        if math.isnan(g):
            continue
        assert np.signbit(g) and abs(g) < 6e-9, (z, g)
        worst = max(worst, abs(float(g)))
    assert worst > 5e-9          # the bound is approached just beyond 6
    # the exact treatment's magnitudes there: |z| Q(|z|) <= 6 Q(6)
    assert 6 * 0.5 * math.erfc(6 / math.sqrt(2)) < 6e-9


def test_nan_only_where_the_expansion_overflows():
    zs = grid()
    nan_at = [z for z in zs if math.isnan(first_pass_gelu(z)) or math.isnan(first_pass_gelu(-z))]
    assert nan_at and min(nan_at) > 1e9
    assert math.isnan(first_pass_gelu(F(np.inf))) and math.isnan(first_pass_gelu(F(np.nan)))


def test_scale_byte_threshold_covers_the_tail_values():
    # a block whose scale byte S is at least 103 has amax >= 2^(S - 125) >= 2^-22
    # and scale 2^(S - 127) >= 2^-24: values below 0.25 scale round to a zero code
    assert 6e-9 < 0.25 * 2.0 ** -24 and 6e-9 < 2.0 ** -22
