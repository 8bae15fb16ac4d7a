"""Stage 2's BF16 regeneration of the selected seeds, and the FP4 step-count
ablation.

The project page ("Two-Stage Pipeline") and the aitrends summary (Stage-2
paragraph) describe the other side of the seed filter: the K = 24 seeds that
the FP4 exploration keeps (top and bottom 12 of 96) are regenerated in BF16
with the full step budget, and those samples train the policy. The aitrends
summary's ablation paragraph reports that ranking with few FP4 steps already
agrees with the full-budget ranking, saturating at about 6 steps.

Here, on the synthetic velocity network of the exploration stage:
  * bf16_velocity: the same 4-block residual MLP with BF16 linears (torch's
    bf16 GEMM, fp32 accumulation, bf16 outputs), RMSNorm and GELU in fp32;
  * Bf16Regenerator: integrates given seeds with that network on the uniform
    grid t_i = 1 - i / steps, the Euler update and the proxy reward through
    this library's kernels (euler_step, fp4_proxy_reward);
  * step_ablation: FP4 rollouts of all candidates with S = 2 .. 10 steps
    ranked against a BF16 rollout with the full step budget (Spearman rho,
    Kendall tau, top/bottom-K overlap).
The BF16 linears are plain library GEMMs (the pages' BF16 path); no FP4
arithmetic happens here.
"""
import time

import numpy as np

from . import binding as fb


def bf16_velocity(x, w1, w2, eps=1e-6):
    """v(x) = h_4, h_{b+1} = h_b + W2_b GELU(W1_b RMSNorm(h_b)), with the two
    linears in bf16 (inputs rounded to bf16, fp32 accumulation, bf16 output)
    and RMSNorm, GELU and the residual sum in fp32. x: fp32 [rows, dim]."""
    import torch
    import torch.nn.functional as F
    h = x.clone()
    for a, b in zip(w1, w2):
        y = h * torch.rsqrt(h.pow(2).mean(-1, keepdim=True) + eps)
        z = F.gelu(F.linear(y.bfloat16(), a).float())
        h = h + F.linear(z.bfloat16(), b).float()
    return h


class Bf16Regenerator:
    """BF16 regeneration of seeds: w1[b] [hidden, dim], w2[b] [dim, hidden]
    (bf16 CUDA tensors), u fp32 [dim] (the proxy reward's vector)."""

    def __init__(self, w1, w2, u, chunk=8):
        self.w1 = [w.bfloat16() for w in w1]
        self.w2 = [w.bfloat16() for w in w2]
        self.u = u
        self.chunk = chunk

    def run(self, noise, steps):
        """noise: fp32 [n, tokens, dim]. Returns (x_final [n, tokens, dim],
        rewards [n]); noise is left intact."""
        import torch
        n, tokens, dim = noise.shape
        x = noise.reshape(n * tokens, dim).clone()
        v = torch.empty_like(x)
        t = [1.0 - i / steps for i in range(steps + 1)]
        for i in range(steps):
            for c0 in range(0, n, self.chunk):
                rows = slice(c0 * tokens, min(n, c0 + self.chunk) * tokens)
                v[rows] = bf16_velocity(x[rows], self.w1, self.w2)
            fb.euler(x, v, t[i], t[i + 1], out=x)
        rewards = fb.proxy_reward(x, n, tokens, self.u)
        return x.view(n, tokens, dim), rewards

    def regenerate(self, noise, seeds, steps):
        """Regenerate the candidates `seeds` (int indices into noise's first
        axis, e.g. the concatenated top and bottom lists of the FP4
        exploration) with `steps` BF16 steps."""
        import torch
        idx = torch.as_tensor(seeds, device=noise.device).long()
        return self.run(noise.index_select(0, idx).contiguous(), steps)


def rank_stats(a, b, k):
    """Agreement of two reward vectors: Spearman rho, Kendall tau (pairs of
    distinct values), and the overlap of their top-k and bottom-k sets."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    ra, rb = np.argsort(np.argsort(a)), np.argsort(np.argsort(b))
    rho = float(np.corrcoef(ra, rb)[0, 1])
    n = len(a)
    conc = 0.0
    for i in range(n):
        conc += float(np.sum(np.sign(a[i] - a[i + 1:]) * np.sign(b[i] - b[i + 1:])))
    tau = conc / (n * (n - 1) / 2)
    ta, tb = set(np.argsort(-a)[:k]), set(np.argsort(-b)[:k])
    ba, bb = set(np.argsort(a)[:k]), set(np.argsort(b)[:k])
    return {"spearman": round(rho, 4), "kendall_tau": round(tau, 4), "top_overlap": len(ta & tb),
            "bottom_overlap": len(ba & bb), "k": k}


def _timed(fn):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out = fn()
    torch.cuda.synchronize()
    return out, time.perf_counter() - t0


def step_ablation(noise, w1, w2, u, k_top, k_bottom, fp4_steps=(2, 4, 6, 10), ref_steps=20, explore_steps=6,
                  chunk=None, bf16_chunk=8):
    """Rank agreement of FP4 explorations with S steps against a BF16
    rollout of every candidate with ref_steps steps, then the BF16
    regeneration of the seeds that the explore_steps FP4 exploration keeps.
    Synthetic weights: the figures describe this network, not a trained
    transformer. Returns a dict (times in seconds)."""
    from .rollout import Fp4Rollout
    regen = Bf16Regenerator(w1, w2, u, chunk=bf16_chunk)
    (_, r_ref), t_ref = _timed(lambda: regen.run(noise, ref_steps))
    r_ref = r_ref.cpu().numpy()
    out = {"reference": {"kind": "bf16 linears", "steps": ref_steps, "seconds": round(t_ref, 3)}, "fp4": {}}
    import torch
    work = torch.empty_like(noise)
    sel = None
    for s in fp4_steps:
        ro = Fp4Rollout(w1, w2, u, steps=s, k_top=k_top, k_bottom=k_bottom, chunk=chunk)
        ro.run(noise, work)  # warm: weights quantized, buffers allocated
        (r, top, bottom, _), t_s = _timed(lambda: ro.run(noise, work))
        out["fp4"][str(s)] = {"seconds": round(t_s, 3), **rank_stats(r.cpu().numpy(), r_ref, k_top)}
        if s == explore_steps:
            sel, t_explore = torch.cat([top, bottom]), t_s
    if sel is not None:
        (_, _), t_regen = _timed(lambda: regen.regenerate(noise, sel, ref_steps))
        out["stage2_regeneration"] = {"seeds": int(sel.numel()), "bf16_steps": ref_steps,
                                      "seconds": round(t_regen, 3), "fp4_exploration_seconds": round(t_explore, 3),
                                      "fp4_exploration": f"{noise.shape[0]} seeds x {explore_steps} steps"}
    return out
