"""Stage 2's BF16 regeneration (fp4_quantized_diffusion_amd.stage2) against
the oracle's rollout with unquantized linears (oracle.rollout, fmt=None: the
same network in float64 with fp32 linear inputs).

* One residual block evaluated once, element by element, within a bound
  derived from the BF16 path's roundings: the linear inputs and outputs are
  rounded to bf16 (relative 2^-9 each), the products accumulate in fp32
  (K 2^-24 of sum |a b|), GELU is 1.13-Lipschitz. With y = RMSNorm(x),
  z = W1 y, g = GELU(z) (all exact):
      |dz| <= 2^-9 (|W1| |y| + |z|) + K1 2^-24 |W1| |y|
      |dg| <= 1.13 |dz| + 2^-9 |g|
      |dh| <= |W2| |dg| + 2^-9 (|W2| |g| + |W2 g|) + K2 2^-24 |W2| |g| + 2^-24 |h|
  taken with a factor 1.5 for the second-order terms.
* A full regeneration (4 blocks, 10 steps): statistical only (the bound
  compounds through the network), final-latent relative error and reward
  agreement within the recorded margin.
"""
import numpy as np
import pytest
import torch

from fp4_quantized_diffusion_amd import inputs, stage2
from oracle import reward as oreward, rollout as orollout
from tests._parity import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -9
E = 2.0 ** -24


def bf16_weights(seed, blocks, dim, hidden):
    ws = [inputs.rollout_weights(seed, b, dim, hidden) for b in range(blocks)]
    w1 = [torch.from_numpy(w[0]).to(DEV).bfloat16() for w in ws]
    w2 = [torch.from_numpy(w[1]).to(DEV).bfloat16() for w in ws]
    return w1, w2


def test_one_block_within_bf16_bound(gpu_lib):
    rows, dim, hidden = 512, 256, 1024
    w1, w2 = bf16_weights(12, 1, dim, hidden)
    x = np.random.default_rng(12).standard_normal((rows, dim)).astype(np.float32)
    h_gpu = to_np(stage2.bf16_velocity(torch.from_numpy(x).to(DEV), w1, w2)).astype(np.float64)
    W1 = to_np(w1[0].float()).astype(np.float64)
    W2 = to_np(w2[0].float()).astype(np.float64)
    l1 = orollout.QuantLinear(W1.astype(np.float32), None)
    l2 = orollout.QuantLinear(W2.astype(np.float32), None)
    h_or = orollout.velocity(x, [l1], [l2])
    y = orollout.rmsnorm(x)
    z = y @ W1.T
    g = orollout.gelu(z)
    ayw = np.abs(y) @ np.abs(W1).T
    dz = U * (ayw + np.abs(z)) + dim * E * ayw + 2.0 ** -20 * ayw
    dg = 1.13 * dz + U * np.abs(g) + 1e-6 * np.abs(g)
    agw = np.abs(g) @ np.abs(W2).T
    dh = dg @ np.abs(W2).T + U * (agw + np.abs(g @ W2.T)) + hidden * E * agw + E * np.abs(h_or)
    err = np.abs(h_gpu - h_or)
    ratio = err / (1.5 * dh)
    print(f"one block: max err / bound {ratio.max():.3f}, mean {ratio.mean():.4f}")
    assert (ratio <= 1).all(), ratio.max()


# Observed on MI355X (seed 13, 6 seeds x 64 tokens, dim 256, hidden 1024, 4
# blocks, 10 steps): final-latent relative L2 7.2e-4, largest reward error
# 7.8e-4 of the largest reward; the gates leave about twice that.
def test_regeneration_against_oracle(gpu_lib):
    seed, n, tokens, dim, hidden, steps = 13, 6, 64, 256, 1024, 10
    noise = np.stack([inputs.rollout_noise(seed, c, tokens, dim) for c in range(n)])
    w1, w2 = bf16_weights(seed, 4, dim, hidden)
    u = inputs.reward_vector(seed, dim)
    regen = stage2.Bf16Regenerator(w1, w2, torch.from_numpy(u).to(DEV), chunk=4)
    nd = torch.from_numpy(noise).to(DEV)
    x_gpu, r_gpu = regen.run(nd, steps)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(nd), noise)  # the seeds' noise is left intact
    w1f = [to_np(w.float()) for w in w1]
    w2f = [to_np(w.float()) for w in w2]
    x_or, r_or, _, _ = orollout.rollout(noise, w1f, w2f, u, n_steps=steps, fmt=None, k_top=1, k_bottom=1)
    xg = to_np(x_gpu).astype(np.float64)
    rel = np.linalg.norm(xg - x_or) / np.linalg.norm(x_or)
    rrel = np.abs(to_np(r_gpu) - r_or).max() / np.abs(r_or).max()
    print(f"regeneration: final-latent rel L2 {rel:.3e}, reward rel {rrel:.3e}")
    assert rel < 1.5e-3 and rrel < 1.6e-3
    # the proxy reward is that of the GPU's own final state (float64 oracle of it)
    want = oreward.proxy_reward(xg.reshape(n * tokens, dim), tokens, u)
    np.testing.assert_allclose(to_np(r_gpu), want, rtol=1e-5, atol=1e-6 * np.abs(want).max())


def test_regenerate_selected_seeds_equals_run_on_them(gpu_lib):
    """regenerate(noise, seeds) is run() on the chosen candidates, bit for bit
    (each candidate's rows are independent of the others)."""
    seed, n, tokens, dim, hidden = 14, 7, 32, 256, 512
    noise = torch.from_numpy(np.stack([inputs.rollout_noise(seed, c, tokens, dim) for c in range(n)])).to(DEV)
    w1, w2 = bf16_weights(seed, 2, dim, hidden)
    u = torch.from_numpy(inputs.reward_vector(seed, dim)).to(DEV)
    regen = stage2.Bf16Regenerator(w1, w2, u, chunk=3)
    seeds = torch.tensor([5, 0, 3], dtype=torch.int32, device=DEV)
    xa, ra = regen.regenerate(noise, seeds, 4)
    xb, rb = regen.run(noise[[5, 0, 3]].contiguous(), 4)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(xa), to_np(xb))
    np.testing.assert_array_equal(to_np(ra), to_np(rb))
