"""Block-scaled FP4 x FP4 GEMM -- oracle, test infrastructure only.

The rollout linear of the FP4 solver (Sol-RL project page, "Two-Stage
Pipeline": FP4 solver at up to 4x the BF16 rate) multiplies FP4 activations by
FP4 weights with a wide accumulator. Plain definition used here:

    C[m, n] = sum_k A_hat[m, k] * B_hat[n, k]

with A_hat, B_hat the exactly dequantized operands (B in nn.Linear layout
[N, K]). MXFP4 products have <= 2+2 significant bits times a power of two and
are exact in float64; the float64 sum then errs by at most K 2^-53 S_abs, far
below the 1e-4 S_abs tolerance. For the NVFP4-style format the per-element
factor G[m] dec(S) has <= 6 significant bits, so those products are exact too;
the two fp32 tensor scales multiply the float64 sum once at the end.

Also returned: S_abs[m, n] = sum_k |A_hat[m, k]| |B_hat[n, k]|, the scale of the
tolerance |C_gpu - C| <= 1e-4 S_abs.
"""
import numpy as np

from . import mxfp4, nvfp4


def gemm_dense(a_hat, b_hat):
    """C = A_hat B_hat^T and S_abs, float64."""
    a_hat = np.asarray(a_hat, dtype=np.float64)
    b_hat = np.asarray(b_hat, dtype=np.float64)
    return a_hat @ b_hat.T, np.abs(a_hat) @ np.abs(b_hat).T


def gemm_mx(a_codes, a_scales, b_codes, b_scales):
    return gemm_dense(mxfp4.dequant(a_codes, a_scales), mxfp4.dequant(b_codes, b_scales))


def gemm_nv(a_codes, a_scales, a_sg, b_codes, b_scales, b_sg):
    c, s = gemm_dense(nvfp4.dequant_unscaled(a_codes, a_scales),
                      nvfp4.dequant_unscaled(b_codes, b_scales))
    g = np.float64(np.float32(a_sg)) * np.float64(np.float32(b_sg))
    return c * g, s * g
