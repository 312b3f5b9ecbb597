"""Flow-matching Euler sampler update ("Cosmos 3 方法原理全解" §7.2).

    x_next = x + (sigma_next - sigma) * v,   sigma_next < sigma,

so integration runs from noise (sigma = 1) towards data (sigma = 0).  The
sigmas are the float32 values handed to the kernel, upcast to float64.

§6.3 gives the rectified-flow path x_sigma = sigma*eps + (1 - sigma)*x0 with
the constant true velocity v* = eps - x0; on that path the Euler update is
exact, which is what pins this function (see the tests).
"""
from __future__ import annotations

import numpy as np


def step(x, v, sigma: float, sigma_next: float) -> np.ndarray:
    s = np.float64(np.float32(sigma))
    sn = np.float64(np.float32(sigma_next))
    return np.asarray(x, dtype=np.float64) + (sn - s) * np.asarray(v, dtype=np.float64)


def flow_path(eps, x0, sigma: float) -> np.ndarray:
    """x_sigma = sigma*eps + (1 - sigma)*x0 (§6.3)."""
    s = np.float64(sigma)
    return s * np.asarray(eps, np.float64) + (1.0 - s) * np.asarray(x0, np.float64)


def true_velocity(eps, x0) -> np.ndarray:
    """v* = eps - x0 (§6.3)."""
    return np.asarray(eps, np.float64) - np.asarray(x0, np.float64)


def linear_schedule(n_steps: int):
    """sigma_k = 1 - k/n, k = 0..n (reading: 'linear' with no shift)."""
    return [1.0 - k / n_steps for k in range(n_steps + 1)]
