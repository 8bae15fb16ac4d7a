"""Comparison helpers for the GPU parity tests (no GPU needed to import)."""
import numpy as np

from oracle import e2m1, mxfp4, nvfp4


def to_np(t):
    return t.detach().cpu().numpy()


def gemm_within_tol(c_gpu, c_exact, s_abs, bf16_out=False, rel=1e-4):
    """|C_gpu - C| <= 1e-4 S_abs (+ one bf16 rounding of C for bf16 output)
    (+ the fp32 underflow floor)."""
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    tol = rel * s_abs + 1e-38
    if bf16_out:
        tol = tol + 2.0 ** -8 * np.abs(c_exact)
    err = np.abs(c_gpu - c_exact)
    bad = err > tol
    return (not bad.any()), float((err / np.maximum(tol, 1e-300)).max())


def mx_codes_near_boundary_ok(x_ref, gpu_codes, gpu_scales, rel=2e-6, band=None):
    """Codes/scales of a quantizer whose input the GPU computes in fp32 (a
    fused prologue) against the float64 reference input x_ref: every code and
    scale must equal the oracle's, except where x_ref sits within `rel`
    (relative) -- plus `band` (absolute, per element, when given: a bound on
    the GPU's fp32 evaluation error) -- of a decision point (a scale binade
    edge for the block max, or an E2M1 threshold); there either neighbour is a
    valid result.
    Returns (n_exact_mismatch_outside_tolerance, n_boundary_flips)."""
    x_ref = np.asarray(x_ref, dtype=np.float64)
    rows, k = x_ref.shape
    oc, os_ = mxfp4.quantize(x_ref.astype(np.float32))
    gn = e2m1.unpack(gpu_codes[:, : k // 2])
    on = e2m1.unpack(oc)
    gs = np.asarray(gpu_scales[:, : k // 32]).astype(np.int64)
    osc = os_.astype(np.int64)
    bad = 0
    flips = 0
    xb = x_ref.reshape(rows, k // 32, 32)
    amax = np.abs(xb).max(-1)
    band = np.zeros_like(x_ref) if band is None else np.broadcast_to(np.asarray(band, dtype=np.float64), x_ref.shape)
    bmax = band.reshape(rows, k // 32, 32).max(-1)
    # scale: may differ by one only when amax is within the tolerance of a power of two
    ds = gs != osc
    if ds.any():
        l2 = np.log2(np.maximum(amax, 1e-300))
        p2 = np.exp2(np.round(l2))
        near_pow2 = (np.abs(l2 - np.round(l2)) < rel * 2) | (np.abs(amax - p2) <= bmax)
        okay = ds & near_pow2 & (np.abs(gs - osc) == 1)
        bad += int((ds & ~okay).sum())
        flips += int(okay.sum())
    # codes: compare where scales agree
    same = np.repeat(gs == osc, 32, axis=1)
    dc = (gn != on) & same
    if dc.any():
        E = np.repeat(osc - 127, 32, axis=1)
        y = np.abs(np.ldexp(x_ref, -E))
        yb = np.ldexp(band, -E)
        thr = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
        slack = np.min(np.abs(y[..., None] - thr) - rel * thr - yb[..., None], axis=-1)
        adjacent = np.abs((gn & 7).astype(int) - (on & 7).astype(int)) == 1
        okay_mag = (slack < 0) & adjacent & ((gn & 8) == (on & 8))
        # the sign (decision point 0) may differ only for a value within the band of zero
        okay_sign = (band > 0) & (np.abs(x_ref) <= band) & ((gn & 7) == 0) & ((on & 7) == 0)
        okay = dc & (okay_mag | okay_sign)
        bad += int((dc & ~okay).sum())
        flips += int(okay.sum())
    return bad, flips


def nv_codes_near_boundary_ok(x_ref, gpu_codes, gpu_scales, sg, rel=2e-6, band=None):
    """The NVFP4-style counterpart of mx_codes_near_boundary_ok, for tensor
    scale sg: every E4M3 scale and code must equal the oracle's for the
    float64 reference input x_ref, except where x_ref sits within `rel`
    (relative) plus `band` (absolute, per element) of a decision point -- an
    E4M3 rounding midpoint for the block amax over fl(6 sg), or an E2M1
    threshold for x over the block's divisor; there either neighbour is a
    valid result. Returns (n_mismatch_outside_tolerance, n_boundary_flips)."""
    x_ref = np.asarray(x_ref, dtype=np.float64)
    rows, k = x_ref.shape
    sg = np.float32(sg)
    oc, os_, _ = nvfp4.quantize(x_ref.astype(np.float32), s_g=sg)
    gn = e2m1.unpack(gpu_codes[:, : k // 2])
    on = e2m1.unpack(oc)
    gs = np.asarray(gpu_scales[:, : k // 16]).astype(np.int64)
    osc = os_.astype(np.int64)
    band = np.zeros_like(x_ref) if band is None else np.broadcast_to(np.asarray(band, dtype=np.float64), x_ref.shape)
    amax = np.abs(x_ref.reshape(rows, k // 16, 16)).max(-1)
    bmax = band.reshape(rows, k // 16, 16).max(-1)
    tau = float(np.float32(np.float32(6.0) * sg))
    vals = nvfp4.e4m3_values()
    bad = flips = 0
    ds = gs != osc
    if ds.any():
        lo = np.clip(np.minimum(gs, osc), 0, 125)
        mid = (vals[lo] + vals[lo + 1]) / 2
        near = np.abs(amax / tau - mid) * tau <= bmax + rel * amax
        okay = ds & (np.abs(gs - osc) == 1) & near
        bad += int((ds & ~okay).sum())
        flips += int(okay.sum())
    same = np.repeat(gs == osc, 16, axis=1)
    dc = (gn != on) & same
    if dc.any():
        d = np.repeat((vals[osc].astype(np.float32) * sg).astype(np.float32).astype(np.float64), 16, axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            y = np.where(d > 0, np.abs(x_ref) / d, 0.0)
            yb = np.where(d > 0, band / d, 0.0)
        thr = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
        slack = np.min(np.abs(y[..., None] - thr) - rel * thr - yb[..., None], axis=-1)
        adjacent = np.abs((gn & 7).astype(int) - (on & 7).astype(int)) == 1
        okay_mag = (slack < 0) & adjacent & ((gn & 8) == (on & 8))
        okay_sign = (band > 0) & (np.abs(x_ref) <= band) & ((gn & 7) == 0) & ((on & 7) == 0)
        okay = dc & (okay_mag | okay_sign)
        bad += int((dc & ~okay).sum())
        flips += int(okay.sum())
    return bad, flips


def lora_merge_band(w, b, a, scale):
    """Bound on |fp32 LoRA merge - exact| for the GPU's evaluation order
    (rank fmas into acc, then fma(scale, acc, w); every input exact in fp32):
    (rank + 2) 2^-24 (|W| + |scale| |B| |A|)."""
    w, b, a = (np.abs(np.asarray(t, dtype=np.float64)) for t in (w, b, a))
    return (b.shape[1] + 2) * 2.0 ** -24 * (w + abs(float(scale)) * (b @ a))


def panel_to_rows(codes, scales, rows, k):
    """Row-major (codes [rows, k/2], scales [rows, k/32]) of a panel-layout
    MXFP4 operand, plus its padding (codes and scale bytes past rows / k) for
    the padding checks. The layout is the storage order declared with
    FP4_LAYOUT_PANEL in include/fp4rollout.h: (panel of 256 rows, chunk of 128
    elements) blocks, 256 x 64 code bytes and 256 x 4 scale bytes each."""
    codes, scales = np.asarray(codes), np.asarray(scales)
    p, nc = (rows + 255) // 256, (k + 127) // 128
    assert codes.size == p * nc * 16384 and scales.size == p * nc * 1024
    c = codes.reshape(p, nc, 256, 64).transpose(0, 2, 1, 3).reshape(p * 256, nc * 64)
    s = scales.reshape(p, nc, 256, 4).transpose(0, 2, 1, 3).reshape(p * 256, nc * 4)
    pad = dict(code_rows=c[rows:], code_cols=c[:rows, k // 2:], scale_rows=s[rows:], scale_cols=s[:rows, k // 32:])
    return c[:rows, : k // 2], s[:rows, : k // 32], pad
