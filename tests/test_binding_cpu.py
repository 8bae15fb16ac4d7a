"""CPU tests of the torch helpers' argument checks: a malformed output,
residual or input must raise ValueError before anything reaches the library
(the tensors here live on the CPU, so a call that got through would fail in
the library instead)."""
import pytest
import torch

from fp4_quantized_diffusion_amd import binding as fb


def qt(rows, k=64):
    return fb.QTensor(torch.zeros(rows, k // 2, dtype=torch.uint8), torch.zeros(rows, k // 32, dtype=torch.uint8),
                      None, fb.FMT_MX, k)


@pytest.mark.parametrize("out_dtype,out,residual", [
    ("f32", torch.zeros(8, 10), None),                                   # wrong shape
    ("f32", torch.zeros(12, 8).t(), None),                               # inner stride not 1
    ("bf16", torch.zeros(8, 12), None),                                  # dtype does not match out_dtype
    ("f32", torch.zeros(8, 12, dtype=torch.bfloat16), None),
    ("f16", torch.zeros(8, 12), None),                                   # unknown out dtype
    ("bf16", torch.zeros(8, 12, dtype=torch.bfloat16), torch.zeros(8, 12)),  # residual with bf16 out
    ("f32", torch.zeros(8, 16)[:, :12], torch.zeros(8, 12)),             # residual row stride != out's
    ("f32", torch.zeros(8, 12), torch.zeros(8, 10)),                     # residual shape
    ("f32", torch.zeros(8, 12), torch.zeros(8, 12, dtype=torch.float64)),  # residual dtype
])
def test_gemm_rejects_bad_out_or_residual(out_dtype, out, residual):
    with pytest.raises(ValueError):
        fb.gemm(qt(8), qt(12), out_dtype, residual=residual, out=out)


@pytest.mark.parametrize("x,v,out", [
    (torch.zeros(16), torch.zeros(12), None),                     # numel mismatch
    (torch.zeros(4, 8).t(), torch.zeros(32), None),               # x not contiguous
    (torch.zeros(16), torch.zeros(8, 4).t()[:, :2], None),        # v not contiguous
    (torch.zeros(16), torch.zeros(16), torch.zeros(15)),          # out numel
    (torch.zeros(16, dtype=torch.bfloat16), torch.zeros(16), None),  # x must be fp32
])
def test_euler_rejects(x, v, out):
    with pytest.raises(ValueError):
        fb.euler(x, v, 1.0, 0.5, out=out)


@pytest.mark.parametrize("x,n_cand,rows,u,out", [
    (torch.zeros(12, 8), 2, 4, None, None),                       # 12 rows != 2 * 4
    (torch.zeros(8, 8).t(), 2, 4, None, None),                    # inner stride
    (torch.zeros(8, 8, dtype=torch.float64), 2, 4, None, None),   # dtype
    (torch.zeros(8, 8), 2, 4, torch.zeros(6), None),              # u length
    (torch.zeros(8, 8), 2, 4, None, torch.zeros(3)),              # out length
])
def test_proxy_reward_rejects(x, n_cand, rows, u, out):
    with pytest.raises(ValueError):
        fb.proxy_reward(x, n_cand, rows, u=u, out=out)
