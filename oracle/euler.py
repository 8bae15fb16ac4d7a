"""Euler step of the deterministic sampler -- oracle, test infrastructure only.

The FP4 exploration runs an ODE sampler for 6 steps (aitrends summary, Stage-1
paragraph; the project page's "Key Insight" stresses the ODE's determinism).
The pages name no integrator; the reading here is explicit Euler on a uniform
grid from t = 1 (noise) to t = 0:

    t_i = 1 - i / n_steps,   x_{i+1} = x_i + (t_{i+1} - t_i) v_i
"""
import numpy as np


def schedule(n_steps=6):
    """The n_steps+1 grid points as the fp32 values handed to the device."""
    return [np.float32(1.0 - i / n_steps) for i in range(n_steps + 1)]


def step(x, v, t_cur, t_next):
    """x + (t_next - t_cur) v in float64 from the given (fp32) inputs."""
    dt = np.float64(t_next) - np.float64(t_cur)
    return np.asarray(x, dtype=np.float64) + dt * np.asarray(v, dtype=np.float64)
