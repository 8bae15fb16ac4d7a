"""Seeded synthetic inputs shaped like the rollout linears' workloads.

Holds no arithmetic of the method: only random draws, casts and the shapes of
the workloads. The trained diffusion transformers and reward models the pages
use are not available, so these draws stand in for their activations,
weights and noises.

Recipe:
  * numpy.random.default_rng(seed); normal draws are made directly in
    float32 (numpy's float32 ziggurat) and scaled in float32; Student-t draws
    are float64 cast to float32; where a workload is bf16 the float32 values
    are rounded to bf16 (nearest even) and returned as float32 arrays whose
    values are exactly bf16;
  * weights ~ N(0, std 0.02); "outliers x20": round(0.001 numel) positions,
    drawn without replacement, multiplied by 20;
  * activations ~ N(0, 1), or Student-t with 4 degrees of freedom (unscaled);
  * rollout: candidate c's noise from default_rng([seed, c]), block b's
    weights from default_rng([seed, 1000 + b]) (W1 then W2), the reward
    vector from default_rng([seed, 9999]).
  * timing-only inputs (class_linear_device): the same distributions drawn
    on the GPU with torch's generator, for full-size timing runs where the
    numpy draw would take minutes; their values differ from the numpy draw
    and no parity check uses them. Student-t(4) is drawn as
    Z0 / sqrt((Z1^2 + ... + Z4^2) / 4) with independent standard normals.
"""
import numpy as np

# workload shapes: M = candidates x tokens per candidate, and the two linears
# timed per class as (name, K, N): SANA-class its attention QKV projection
# (hidden -> 3 hidden) and MLP down projection, FLUX.1- and SD3.5-L-class
# their MLP up and down projections
CLASS_SHAPES = {
    "sana": dict(m=96 * 1024, hidden=2240, mlp=5600, seed=1, act="normal",
                 gemms=(("qkv", 2240, 6720), ("down", 5600, 2240))),
    "flux": dict(m=8 * 4608, hidden=3072, mlp=12288, seed=2, act="normal",
                 gemms=(("up", 3072, 12288), ("down", 12288, 3072))),
    "sd35": dict(m=8 * 4352, hidden=2432, mlp=9728, seed=3, act="student_t",
                 gemms=(("up", 2432, 9728), ("down", 9728, 2432))),
}


def class_gemm(name, which):
    """(label, K, N) of linear `which` (1 or 2) of a workload class."""
    return CLASS_SHAPES[name]["gemms"][which - 1]

ROLLOUT = dict(n_cand=96, tokens=4096, dim=3072, hidden=12288, blocks=4, steps=6,
               k_top=12, k_bottom=12, seed=4)


def to_bf16(x):
    """float32 -> nearest-even bf16, returned as float32 holding bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    # finite inputs cannot wrap: the largest finite pattern + 0x8000 < 2^32
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    out = rounded.view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = np.where(nan, x, out)
    return out


def bf16_bits(x):
    """float32 array of bf16 values -> uint16 bit patterns."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def weights(rng, out_f, in_f, outliers=True, bf16=True):
    w = rng.standard_normal((out_f, in_f), dtype=np.float32)
    w *= np.float32(0.02)
    if outliers:
        n = int(round(0.001 * w.size))
        pos = rng.choice(w.size, size=n, replace=False)
        w.reshape(-1)[pos] *= np.float32(20.0)
    return to_bf16(w) if bf16 else w


def activations(rng, rows, cols, kind="normal", bf16=True):
    if kind == "student_t":
        a = rng.standard_t(4, size=(rows, cols)).astype(np.float32)
    else:
        a = rng.standard_normal((rows, cols), dtype=np.float32)
    return to_bf16(a) if bf16 else a


def tiny(seed=0):
    """X [128, 256] ~ N(0,1) fp32, W [256, 512] ~ N(0, 0.02) fp32, B = W^T [512, 256]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((128, 256), dtype=np.float32)
    w = rng.standard_normal((256, 512), dtype=np.float32) * np.float32(0.02)
    return x, np.ascontiguousarray(w.T)


def class_linear(name, which, rows=None):
    """Activation [M, K] and weight [N, K] for linear `which` (1 or 2, see
    CLASS_SHAPES) of a workload class. `rows` limits M (the draw of the
    first rows is the same for any limit)."""
    cfg = CLASS_SHAPES[name]
    _, k, n = class_gemm(name, which)
    m = cfg["m"] if rows is None else rows
    rng_w = np.random.default_rng([cfg["seed"], which, 1])
    w = weights(rng_w, n, k)
    rng_a = np.random.default_rng([cfg["seed"], which, 0])
    a = activations(rng_a, m, k, cfg["act"])
    return a, w


def class_linear_device(name, which, device, draw=0, chunk_rows=8192):
    """Like class_linear, drawn on `device` with torch's generator (seeded
    from the class seed, `which` and `draw`): bf16 activation [M, K] and bf16
    weight [N, K]."""
    import torch
    cfg = CLASS_SHAPES[name]
    _, k, n = class_gemm(name, which)
    m = cfg["m"]
    g = torch.Generator(device=device)
    g.manual_seed(cfg["seed"] * 1000003 + which * 1009 + draw)
    w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32) * 0.02
    n_out = int(round(0.001 * w.numel()))
    pos = torch.randperm(w.numel(), generator=g, device=device)[:n_out]
    w.view(-1)[pos] *= 20.0
    a = torch.empty((m, k), dtype=torch.bfloat16, device=device)
    for r0 in range(0, m, chunk_rows):
        r = min(chunk_rows, m - r0)
        z = torch.randn((r, k), generator=g, device=device, dtype=torch.float32)
        if cfg["act"] == "student_t":
            chi2 = torch.zeros_like(z)
            for _ in range(4):
                chi2 += torch.randn((r, k), generator=g, device=device, dtype=torch.float32) ** 2
            z = z / torch.sqrt(chi2 / 4.0)
        a[r0:r0 + r] = z.to(torch.bfloat16)
    return a, w.to(torch.bfloat16)


def rollout_noise(seed, cand, tokens, dim):
    rng = np.random.default_rng([seed, cand])
    return rng.standard_normal((tokens, dim), dtype=np.float32)


def rollout_noise_all(seed, n_cand, tokens, dim, threads=16):
    """[n_cand, tokens, dim]; each candidate's draw is independent of the
    others (numpy releases the GIL while filling, so threads help)."""
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty((n_cand, tokens, dim), dtype=np.float32)

    def fill(c):
        np.random.default_rng([seed, c]).standard_normal((tokens, dim), dtype=np.float32, out=out[c])

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill, range(n_cand)))
    return out


def rollout_weights(seed, block, dim, hidden):
    """(W1 [hidden, dim], W2 [dim, hidden]) as bf16 values."""
    rng = np.random.default_rng([seed, 1000 + block])
    return weights(rng, hidden, dim), weights(rng, dim, hidden)


def reward_vector(seed, dim):
    return np.random.default_rng([seed, 9999]).standard_normal(dim, dtype=np.float32)


def rewards(seed, n, kind="normal"):
    rng = np.random.default_rng([seed, 777])
    if kind == "ties":
        return rng.integers(-3, 4, size=n).astype(np.float32)
    return rng.standard_normal(n, dtype=np.float32)
