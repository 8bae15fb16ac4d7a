"""fp4_gemm_panel_euler_reward_noalloc (the Euler + reward GEMM epilogue with
its partial sums in the library's own device array) against
fp4_gemm_panel_euler_reward (caller workspace): the same kernels in the same
order, so the new state and the rewards must agree bit for bit -- on two
calls in a row, the second with a smaller problem, so a stale or mis-sized
use of the shared array would show. Both calls go through the C ABI."""
import numpy as np
import pytest
import torch

import fp4_quantized_diffusion_amd as fq
from fp4_quantized_diffusion_amd import binding as fb
from tests._parity import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def case(m, n, k, tokens, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    a = fq.quantize(torch.randn(m, k, device=DEV, generator=g), "mx", layout="panel")
    b = fq.quantize(torch.randn(n, k, device=DEV, generator=g) * 0.05, "mx", layout="panel")
    res = torch.randn(m, n, device=DEV, generator=g)
    x = torch.randn(m, n, device=DEV, generator=g)
    u = torch.randn(n, device=DEV, generator=g)
    return a, b, res, x, u


@pytest.mark.parametrize("shapes", [[(1024, 512, 256, 256), (512, 256, 128, 128)],
                                    [(2048, 768, 384, 512), (256, 256, 256, 128)]])
def test_noalloc_equals_workspace_variant(gpu_lib, shapes):
    for i, (m, n, k, tokens) in enumerate(shapes):
        a, b, res, x, u = case(m, n, k, tokens, 100 + i)
        want_x, want_r = fq.gemm_euler_reward(a, b, res, x, 1.0, 5.0 / 6.0, u, tokens)
        out = torch.full((m, n), float("nan"), device=DEV)
        rewards = torch.full((m // tokens,), float("nan"), device=DEV)
        st = fb.fp4_gemm_panel_euler_reward_noalloc(
            fb.FMT_MX, a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(), b.scales.data_ptr(), m, n, k,
            res.data_ptr(), x.data_ptr(), out.data_ptr(), n, 1.0, 5.0 / 6.0, u.data_ptr(), tokens,
            rewards.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == fb.OK, fb.status_str(st)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(out), to_np(want_x))
        np.testing.assert_array_equal(to_np(rewards), to_np(want_r))
        # the torch helper over the same entry point
        out2, r2 = fq.gemm_euler_reward_noalloc(a, b, res, x, 1.0, 5.0 / 6.0, u, tokens, torch.empty_like(x),
                                                torch.empty(m // tokens, device=DEV))
        np.testing.assert_array_equal(to_np(out2), to_np(want_x))
        np.testing.assert_array_equal(to_np(r2), to_np(want_r))


def test_noalloc_rejects_oversized_problem_before_launch(gpu_lib):
    """(m / 256) (n / 256) 4 above 2^18 partial sums: rejected on the host,
    nothing launched (the small buffers below would not hold such a problem)."""
    a, b, res, x, u = case(256, 256, 128, 128, 7)
    rewards = torch.empty(4, device=DEV)
    st = fb.fp4_gemm_panel_euler_reward_noalloc(
        fb.FMT_MX, a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(), b.scales.data_ptr(), 256 * 512,
        256 * 129, 128, res.data_ptr(), x.data_ptr(), x.data_ptr(), 256 * 129, 1.0, 0.5, u.data_ptr(), 128,
        rewards.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == fb.INVALID_ARGUMENT
