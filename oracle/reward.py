"""Proxy reward, reward normalisation and top/bottom seed selection --
oracle, test infrastructure only.

* Selection (Sol-RL project page, "Two-Stage Pipeline", Stage 1; aitrends
  summary, Stage-1 paragraph): from N = 96 candidates keep K = 24 seeds, the
  K/2 with the highest and the K/2 with the lowest proxy reward.
* Normalisation (VeRL-Omni DiffusionNFT docs, "Algorithm", first equation):
  r = 1/2 + 1/2 clip((r_raw - mean) / Z, -1, 1), Z a standard deviation over
  the batch (global by default).

Readings: Z is the population standard deviation (ddof = 0); Z == 0 gives
r = 1/2 everywhere. Ranking uses the raw reward (r is monotone in it but ties
at the clip limits). One total order -- reward descending, equal rewards by
ascending index -- defines both lists: `top` is its first k_top entries,
`bottom` its last k_bottom entries listed from the lowest reward upward, so
the lists never overlap when k_top + k_bottom <= N.
"""
import numpy as np


def proxy_reward(x, rows_per_cand, u=None):
    """x: [n_cand * rows_per_cand, dim]. Per candidate: the mean over its rows,
    then either the mean over dims (u is None) or the dot product with u."""
    x = np.asarray(x, dtype=np.float64)
    dim = x.shape[-1]
    xc = x.reshape(-1, rows_per_cand, dim)
    mean_rows = xc.mean(axis=1)                      # [n_cand, dim]
    if u is None:
        return mean_rows.mean(axis=1)
    return mean_rows @ np.asarray(u, dtype=np.float64)


def normalize(r):
    r = np.asarray(r, dtype=np.float64)
    mu = r.mean()
    sd = r.std()                                     # ddof = 0
    if sd == 0:
        return np.full_like(r, 0.5)
    return 0.5 + 0.5 * np.clip((r - mu) / sd, -1.0, 1.0)


def order(r):
    """The total order: reward descending, ties by ascending index. Every NaN
    ranks below -inf (NaNs among themselves by index); -0 equals +0. The
    pages assume finite rewards; this convention only makes the order total,
    so that a selection always names valid candidates."""
    r = [float(v) for v in np.asarray(r, dtype=np.float64)]
    return sorted(range(len(r)), key=lambda i: (1, 0.0, i) if r[i] != r[i] else (0, -r[i], i))


def select(r, k_top, k_bottom):
    n = len(r)
    if k_top < 0 or k_bottom < 0 or k_top + k_bottom > n:
        raise ValueError("need 0 <= k_top, k_bottom and k_top + k_bottom <= n")
    o = order(r)
    top = o[:k_top]
    bottom = o[::-1][:k_bottom]
    return np.array(top, dtype=np.int32), np.array(bottom, dtype=np.int32)
