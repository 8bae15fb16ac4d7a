"""LoRA merge of a weight matrix -- oracle, test infrastructure only.

The policy is trained with LoRA adapters of rank 32, and after each update the
adapted weights are re-quantized at run time for the next FP4 rollout, with
no compile step (aitrends summary, Stage-2 paragraph; Sol-RL project page,
"Two-Stage Pipeline", Stage 2). The pages do not spell out the merge; the
reading used here is the standard LoRA form

    W' = W + s (B A),    W [N, K] (nn.Linear layout), B [N, r], A [r, K],

with the scale s (alpha / r in the usual parametrisation) a caller argument.
The re-quantized weight is then mxfp4.quantize(W'), the same rule as for any
other weight.

Arithmetic: float64 with a library matmul for B A. Every product of two fp32
(or bf16) values is exact in float64; the sum of r such products carries at
most about r 2^-53 relative error of sum |B A|, far below anything the fp32
GPU evaluation resolves.
"""
import numpy as np


def merge(w, b, a, scale):
    """W + scale * (B @ A) in float64. w: [N, K]; b: [N, r]; a: [r, K]."""
    w = np.asarray(w, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    if w.ndim != 2 or b.ndim != 2 or a.ndim != 2:
        raise ValueError("w, b and a must be 2-D")
    if b.shape[0] != w.shape[0] or a.shape[1] != w.shape[1] or b.shape[1] != a.shape[0]:
        raise ValueError("shapes do not chain: w [N, K], b [N, r], a [r, K]")
    return w + float(scale) * (b @ a)
