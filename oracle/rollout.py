"""Synthetic FP4 exploration rollout -- oracle, test infrastructure only.

Stage 1 of the two-stage pipeline (Sol-RL project page, "Two-Stage Pipeline";
aitrends summary, Stage-1 paragraph): quantize the current weights to FP4,
integrate N noises with a 6-step ODE solver whose linears run in FP4, score
the candidates with a proxy reward and keep the top K/2 and bottom K/2 seeds.

The pages' velocity network is a trained DiT; this stand-in keeps only the
shape of its MLP linears. Readings (the pages give no network):
  * velocity v(x) = h_4 with h_0 = x and
        h_{b+1} = h_b + W2_b GELU(W1_b RMSNorm(h_b)),   b = 0..3
    RMSNorm with unit gain and eps 1e-6, exact (not tanh-approximated) GELU,
    GELU(z) = z Phi(z) with Phi the standard normal CDF, no time conditioning;
  * every linear input is rounded to fp32 and then quantized (the quantizers
    take fp32 or bf16 input); everything else is float64;
  * the hidden activation z = W1 RMSNorm(h) enters GELU unrounded
    (hidden="f32", the default). hidden="bf16" is the other reading a bf16
    network would take: z rounded to fp32 and then to bf16, both to nearest
    even, before GELU;
  * proxy reward = <mean over tokens of x_final, u> for a fixed vector u;
  * Euler steps on the uniform grid t_i = 1 - i/6.
"""
import numpy as np
from scipy.special import erfc

from . import euler, gemm, mxfp4, nvfp4, reward

EPS = 1e-6


def rmsnorm(h):
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + EPS)


def gelu(z):
    """z Phi(z), Phi(z) = erfc(-z / sqrt 2) / 2: the same function as
    0.5 z (1 + erf(z / sqrt 2)), written so the negative tail keeps its
    relative accuracy (1 + erf cancels there)."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * erfc(-z / np.sqrt(2.0))


class QuantLinear:
    """A weight [out, in] quantized once per iteration (the pages' per-iteration
    re-quantization) and held dequantized (exact float64); __call__ quantizes
    its fp32 input and forms the exact product with that weight."""

    def __init__(self, w, fmt):
        self.fmt = fmt
        w = np.asarray(w, dtype=np.float32)
        if fmt == "mx":
            self.w_hat = mxfp4.dequant(*mxfp4.quantize(w))
        elif fmt == "nv":
            c, s, g = nvfp4.quantize(w)
            self.w_hat = nvfp4.dequant(c, s, g)
        elif fmt is None:
            self.w_hat = w.astype(np.float64)
        else:
            raise ValueError(fmt)

    @classmethod
    def from_quantized(cls, fmt, codes, scales, s_g=None):
        """A layer whose weight is already in quantized form."""
        self = cls.__new__(cls)
        self.fmt = fmt
        self.w_hat = mxfp4.dequant(codes, scales) if fmt == "mx" else nvfp4.dequant(codes, scales, s_g)
        return self

    def __call__(self, x):
        x32 = np.asarray(x, dtype=np.float32)
        if self.fmt == "mx":
            x_hat = mxfp4.dequant(*mxfp4.quantize(x32))
        elif self.fmt == "nv":
            c, s, g = nvfp4.quantize(x32)
            x_hat = nvfp4.dequant(c, s, g)
        else:
            x_hat = x32.astype(np.float64)
        return gemm.gemm_dense(x_hat, self.w_hat)[0]


def bf16_round(z):
    """z rounded to fp32, then to bf16 (8 significant bits), each to nearest
    with ties to even, as float64. The second rounding drops the 16 low bits
    of the fp32 pattern: add half of their range, minus one unless the lowest
    kept bit is set, then clear them (finite inputs; the carry may step into
    the exponent, which is the correct rounding)."""
    f = np.ascontiguousarray(np.asarray(z, dtype=np.float64).astype(np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def velocity(x, w1, w2, hidden="f32"):
    """x: [tokens_total, dim]; w1[b]: QuantLinear dim->hidden; w2[b]: hidden->dim.
    hidden: "f32" (GELU of z itself) or "bf16" (GELU of bf16_round(z))."""
    if hidden not in ("f32", "bf16"):
        raise ValueError(hidden)
    h = np.asarray(x, dtype=np.float64)
    for l1, l2 in zip(w1, w2):
        z = l1(rmsnorm(h))
        if hidden == "bf16":
            z = bf16_round(z)
        h = h + l2(gelu(z))
    return h


def rollout(noise, w1, w2, u, n_steps=6, fmt="mx", k_top=12, k_bottom=12, hidden="f32"):
    """noise: [n_cand, tokens, dim]; w1/w2: lists of float weights [out, in]
    (or of ready QuantLinear layers); hidden: as velocity.

    Returns (x_final [n_cand, tokens, dim], rewards [n_cand], top, bottom)."""
    noise = np.asarray(noise, dtype=np.float32)
    n_cand, tokens, dim = noise.shape
    q1 = [w if isinstance(w, QuantLinear) else QuantLinear(w, fmt) for w in w1]
    q2 = [w if isinstance(w, QuantLinear) else QuantLinear(w, fmt) for w in w2]
    t = euler.schedule(n_steps)
    x = noise.reshape(n_cand * tokens, dim).astype(np.float64)
    for i in range(n_steps):
        v = velocity(x, q1, q2, hidden)
        x = euler.step(x, v, t[i], t[i + 1])
    r = reward.proxy_reward(x, tokens, u)
    top, bottom = reward.select(r, k_top, k_bottom)
    return x.reshape(n_cand, tokens, dim), r, top, bottom
