"""DiffusionNFT training-side pieces -- oracle, test infrastructure only.

The seeds selected by the FP4 rollout are regenerated in BF16 and the policy
is updated with DiffusionNFT (aitrends summary, Stage-2 paragraph; Sol-RL
project page, "Two-Stage Pipeline"). The VeRL-Omni DiffusionNFT docs,
section "Algorithm", define the pieces used here:

  * the optimality probability r from the raw rewards (reward.normalize);
  * forward noising of a clean latent x0 at time t and the flow-matching
    target velocity. Reading: the rectified-flow path of the rollout's
    sampler, x_t = (1 - t) x0 + t eps, whose velocity is v = eps - x0
    (the sampler integrates dx/dt = v from t = 1, noise, to t = 0);
  * the loss, with the implicit branches
        v+ = (1 - beta) v_old + beta v_theta,
        v- = (1 + beta) v_old - beta v_theta,
        L  = mean over samples of  r ||v+ - v||^2 + (1 - r) ||v- - v||^2,
    the squared norm summed over the sample's elements.

Arithmetic: float64, in the order the equations are written.
"""
import numpy as np


def noise(x0, eps, t):
    """x_t = (1 - t) x0 + t eps per sample. x0, eps: [N, ...]; t: [N]."""
    x0 = np.asarray(x0, dtype=np.float64)
    eps = np.asarray(eps, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64).reshape((-1,) + (1,) * (x0.ndim - 1))
    return (1.0 - t) * x0 + t * eps


def target_velocity(x0, eps):
    return np.asarray(eps, dtype=np.float64) - np.asarray(x0, dtype=np.float64)


def loss_terms(v_old, v_theta, x0, eps, r, beta):
    """Per-sample r ||v+ - v||^2 + (1 - r) ||v- - v||^2, [N] float64."""
    v_old = np.asarray(v_old, dtype=np.float64)
    v_theta = np.asarray(v_theta, dtype=np.float64)
    v = target_velocity(x0, eps)
    n = v_old.shape[0]
    vp = (1.0 - beta) * v_old + beta * v_theta
    vn = (1.0 + beta) * v_old - beta * v_theta
    pos = ((vp - v) ** 2).reshape(n, -1).sum(axis=1)
    neg = ((vn - v) ** 2).reshape(n, -1).sum(axis=1)
    r = np.asarray(r, dtype=np.float64)
    return r * pos + (1.0 - r) * neg


def loss(v_old, v_theta, x0, eps, r, beta):
    return float(loss_terms(v_old, v_theta, x0, eps, r, beta).mean())
