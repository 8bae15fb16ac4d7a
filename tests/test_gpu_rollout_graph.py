"""The rollout captured in a HIP graph (Fp4Rollout.graph): every replay, with
new noise written into the captured buffer by eager work between replays,
gives the bytes of an eager rollout of that noise -- the final state, the
rewards, the selection and the normalised rewards. The fused one-stream
path, the unfused path (chunks of 192 and 64 rows) and the two-stream
schedule are each captured."""
import numpy as np
import pytest
import torch

from fp4_quantized_diffusion_amd import inputs
from fp4_quantized_diffusion_amd.rollout import Fp4Rollout

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def weights(dim, hidden, blocks):
    ws = [inputs.rollout_weights(5, b, dim, hidden) for b in range(blocks)]
    w1 = [torch.from_numpy(a).to(DEV).bfloat16() for a, _ in ws]
    w2 = [torch.from_numpy(c).to(DEV).bfloat16() for _, c in ws]
    return w1, w2, torch.from_numpy(inputs.reward_vector(5, dim)).to(DEV)


CASES = {
    # n_cand, tokens, dim, hidden, options
    "fused": (4, 256, 256, 1024, dict()),
    "unfused": (4, 64, 256, 1024, dict(chunk=3)),
    "two_streams": (4, 256, 256, 1024, dict(overlap=True, hidden="bf16")),
}


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_equal_eager_rollouts(case):
    n, tokens, dim, hidden, opts = CASES[case]
    print(f"graph case {case}: {n} x {tokens} x {dim}, hidden {hidden}", flush=True)
    w1, w2, u = weights(dim, hidden, 2)
    mk = lambda: Fp4Rollout(w1, w2, u, steps=3, k_top=1, k_bottom=1, **opts)
    noise = torch.from_numpy(inputs.rollout_noise_all(1, n, tokens, dim)).to(DEV)
    work = torch.empty_like(noise)
    ro = mk()
    replay, (rewards, top, bottom, rn) = ro.graph(noise, work)
    ref = mk()
    for k in range(3):
        fresh = torch.from_numpy(inputs.rollout_noise_all(10 + k, n, tokens, dim)).to(DEV)
        noise.copy_(fresh)                      # eager work between replays
        torch.cuda.synchronize()
        replay()
        torch.cuda.synchronize()
        work_ref = torch.empty_like(fresh)
        r_ref, t_ref, b_ref, rn_ref = ref.run(fresh.clone(), work_ref)
        torch.cuda.synchronize()
        assert torch.equal(work, work_ref), (case, k)
        assert torch.equal(rewards, r_ref) and torch.equal(top, t_ref) and torch.equal(bottom, b_ref), (case, k)
        assert torch.equal(rn, rn_ref), (case, k)
        # the replay saw the new noise, not the captured one
        assert not np.array_equal(rewards.cpu().numpy(), np.zeros(n, np.float32))


def test_graph_refuses_a_timed_rollout():
    w1, w2, u = weights(256, 1024, 1)
    ro = Fp4Rollout(w1, w2, u, steps=1, k_top=1, k_bottom=1, timer=lambda name, fn: fn())
    noise = torch.zeros(2, 256, 256, device=DEV)
    with pytest.raises(ValueError):
        ro.graph(noise)
