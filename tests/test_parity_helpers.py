"""CPU checks of the tolerance helpers the GPU parity tests rely on: the
oracle's own codes pass, a code moved away from an element far from every
decision point is caught, and the allowed flips are only the documented
ones (a neighbour code within the band of a threshold, a neighbour scale
within the band of a rounding midpoint)."""
import numpy as np

from oracle import e2m1, mxfp4, nvfp4
from tests._parity import mx_codes_near_boundary_ok, nv_codes_near_boundary_ok


def nv_case(seed=0, rows=8, k=64):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k))
    sg = nvfp4.tensor_scale(x.astype(np.float32))
    c, s, _ = nvfp4.quantize(x.astype(np.float32), s_g=sg)
    return x, sg, c, s


def test_nv_identity_passes():
    x, sg, c, s = nv_case()
    assert nv_codes_near_boundary_ok(x, c, s, sg) == (0, 0)


def test_nv_code_moved_far_from_threshold_is_caught():
    x, sg, c, s = nv_case(1)
    nib = e2m1.unpack(c)
    # element 0 of row 0 set exactly on a grid value of its block: far from thresholds
    d = np.float32(nvfp4.e4m3_decode(s[0, 0]).astype(np.float32) * sg)
    x = x.copy()
    x[0, 0] = float(np.float32(1.0) * d)
    c, s, _ = nvfp4.quantize(x.astype(np.float32), s_g=sg)
    nib = e2m1.unpack(c)
    nib[0, 0] = (nib[0, 0] & 8) | ((nib[0, 0] & 7) + 1)
    bad, _ = nv_codes_near_boundary_ok(x, e2m1.pack(nib), s, sg)
    assert bad == 1


def test_nv_neighbour_code_within_band_of_threshold_is_a_flip():
    x, sg, c, s = nv_case(2)
    d = float(np.float32(nvfp4.e4m3_decode(s[0, 0]).astype(np.float32) * sg))
    x = x.copy()
    x[0, 1] = 1.25 * d * (1 + 1e-9)  # just above the 1.0 / 1.5 decision point
    c, s, _ = nvfp4.quantize(x.astype(np.float32), s_g=sg)
    nib = e2m1.unpack(c)
    assert nib[0, 1] & 7 in (2, 3)
    nib[0, 1] = (nib[0, 1] & 8) | (5 - (nib[0, 1] & 7))  # the other neighbour
    band = np.zeros_like(x)
    band[0, 1] = 1e-6 * d
    assert nv_codes_near_boundary_ok(x, e2m1.pack(nib), s, sg, band=band) == (0, 1)
    assert nv_codes_near_boundary_ok(x, e2m1.pack(nib), s, sg, rel=0.0)[0] == 1


def test_nv_scale_neighbour_only_at_a_midpoint():
    x, sg, c, s = nv_case(3)
    s2 = s.copy()
    s2[1, 1] = s2[1, 1] + 1
    assert nv_codes_near_boundary_ok(x, c, s2, sg)[0] == 1  # amax not at a midpoint
    vals = nvfp4.e4m3_values()
    tau = float(np.float32(np.float32(6.0) * sg))
    x = x.copy()
    blk = x[1, 16:32]
    i = int(np.argmax(np.abs(blk)))
    mid = (vals[40] + vals[41]) / 2
    blk[i] = np.sign(blk[i]) * mid * tau
    blk[np.arange(16) != i] = np.clip(blk[np.arange(16) != i], -0.5 * mid * tau, 0.5 * mid * tau)
    c, s, _ = nvfp4.quantize(x.astype(np.float32), s_g=sg)
    s2 = s.copy()
    s2[1, 1] = 81 - s[1, 1]  # the other of codes 40 and 41
    bad, flips = nv_codes_near_boundary_ok(x, c, s2, sg)
    assert bad == 0 and flips == 1


def test_mx_identity_and_far_change():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 64))
    c, s = mxfp4.quantize(x.astype(np.float32))
    assert mx_codes_near_boundary_ok(x, c, s) == (0, 0)
    s2 = s.copy()
    s2[0, 0] += 3
    assert mx_codes_near_boundary_ok(x, c, s2)[0] == 1
