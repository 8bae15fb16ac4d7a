"""Comparison helpers for the GPU parity tests (no GPU needed to import)."""
import numpy as np

from oracle import e2m1, mxfp4


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


def mx_codes_near_boundary_ok(x_ref, gpu_codes, gpu_scales, rel=2e-6):
    """Codes/scales of a quantizer whose input the GPU computes in fp32 (a
    fused prologue) against the float64 reference input x_ref: every code and
    scale must equal the oracle's, except where x_ref sits within `rel` of a
    decision point (a scale binade edge for the block max, or an E2M1
    threshold) -- there either neighbour is a valid result.
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
    # scale: may differ by one only when amax is within rel of a power of two
    ds = gs != osc
    if ds.any():
        near_pow2 = np.abs(np.log2(np.maximum(amax, 1e-300)) - np.round(np.log2(np.maximum(amax, 1e-300)))) < rel * 2
        okay = ds & near_pow2 & (np.abs(gs - osc) == 1)
        bad += int((ds & ~okay).sum())
        flips += int(okay.sum())
    # codes: compare where scales agree
    same = np.repeat(gs == osc, 32, axis=1)
    dc = (gn != on) & same
    if dc.any():
        E = np.repeat(osc - 127, 32, axis=1)
        y = np.abs(np.ldexp(x_ref, -E))
        thr = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
        dist = np.min(np.abs(y[..., None] - thr) / thr, axis=-1)
        adjacent = np.abs((gn & 7).astype(int) - (on & 7).astype(int)) == 1
        okay = dc & (dist < rel) & adjacent & ((gn & 8) == (on & 8))
        bad += int((dc & ~okay).sum())
        flips += int(okay.sum())
    return bad, flips


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
