"""Pins for the oracle's block-scaled GEMM (CPU only)."""
from fractions import Fraction

import numpy as np

from oracle import gemm, mxfp4, nvfp4


def nibble_value(nib):
    """E2M1 value from bit fields, as an exact Fraction."""
    s, e, m = (nib >> 3) & 1, (nib >> 1) & 3, nib & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def frac_dequant_mx(codes, scales):
    rows, kb = codes.shape
    out = [[None] * (2 * kb) for _ in range(rows)]
    for r in range(rows):
        for j in range(kb):
            byte = int(codes[r, j])
            for h, nib in enumerate((byte & 15, byte >> 4)):
                k = 2 * j + h
                out[r][k] = nibble_value(nib) * Fraction(2) ** (int(scales[r, k // 32]) - 127)
    return out


def test_exact_rationals_small_mx():
    rng = np.random.default_rng(10)
    for (m, n, k) in [(3, 5, 32), (7, 2, 64), (16, 16, 96)]:
        a = (rng.standard_normal((m, k)) * np.exp(rng.uniform(-3, 3, (m, 1)))).astype(np.float32)
        b = rng.standard_normal((n, k)).astype(np.float32)
        ac, as_ = mxfp4.quantize(a)
        bc, bs = mxfp4.quantize(b)
        c, s = gemm.gemm_mx(ac, as_, bc, bs)
        A, B = frac_dequant_mx(ac, as_), frac_dequant_mx(bc, bs)
        for i in range(m):
            for j in range(n):
                exact = sum(A[i][t] * B[j][t] for t in range(k))
                sabs = sum(abs(A[i][t] * B[j][t]) for t in range(k))
                assert c[i, j] == float(exact)          # exact in float64 at this size
                assert s[i, j] == float(sabs)


def test_exact_rationals_small_nv():
    rng = np.random.default_rng(11)
    m, n, k = 4, 3, 32
    a = rng.standard_normal((m, k)).astype(np.float32)
    b = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    ac, as_, ag = nvfp4.quantize(a)
    bc, bs, bg = nvfp4.quantize(b)
    c, _ = gemm.gemm_nv(ac, as_, ag, bc, bs, bg)
    e4 = nvfp4.e4m3_values()
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for t in range(k):
                na = (int(ac[i, t // 2]) >> (4 * (t % 2))) & 15
                nb = (int(bc[j, t // 2]) >> (4 * (t % 2))) & 15
                tot += (nibble_value(na) * Fraction(e4[as_[i, t // 16]]) *
                        nibble_value(nb) * Fraction(e4[bs[j, t // 16]]))
            tot *= Fraction(float(ag)) * Fraction(float(bg))
            assert abs(c[i, j] - float(tot)) <= 1e-15 * abs(float(tot)) + 1e-300


def test_one_hot_column_and_orientation():
    """A has a single non-zero at (i, t); C row i must equal A[i,t] * B[:, t]."""
    k = 64
    a = np.zeros((4, k), dtype=np.float32)
    a[2, 37] = 3.0
    b = np.arange(5 * k, dtype=np.float32).reshape(5, k) % 7 - 3
    ac, as_ = mxfp4.quantize(a)
    bc, bs = mxfp4.quantize(b)
    c, _ = gemm.gemm_mx(ac, as_, bc, bs)
    bh = mxfp4.dequant(bc, bs)
    np.testing.assert_array_equal(c[2], 3.0 * bh[:, 37])
    assert not c[[0, 1, 3]].any()


def test_identity_weight_returns_activation():
    k = 64
    rng = np.random.default_rng(12)
    a = rng.standard_normal((8, k)).astype(np.float32)
    eye = np.eye(k, dtype=np.float32)
    ac, as_ = mxfp4.quantize(a)
    ec, es = mxfp4.quantize(eye)
    c, _ = gemm.gemm_mx(ac, as_, ec, es)
    np.testing.assert_array_equal(c, mxfp4.dequant(ac, as_))


def test_transpose_symmetry():
    rng = np.random.default_rng(13)
    a = rng.standard_normal((6, 96)).astype(np.float32)
    b = rng.standard_normal((5, 96)).astype(np.float32)
    qa, qb = mxfp4.quantize(a), mxfp4.quantize(b)
    c1, _ = gemm.gemm_mx(*qa, *qb)
    c2, _ = gemm.gemm_mx(*qb, *qa)
    np.testing.assert_allclose(c1, c2.T, rtol=1e-14, atol=0)
