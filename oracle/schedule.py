"""Sampler noise levels with the flow shift.

Sources ("Cosmos 3 方法原理全解"):

* §6.3 defines the shift on a time t in [0, 1]: with t̄ = 1 - t,
  σ = s·t̄ / (1 + (s - 1)·t̄).  It fixes σ = 0 and σ = 1 and, for s > 1,
  pushes every point in between towards high noise.  In odds form it is a
  plain scaling: σ / (1 - σ) = s · t̄ / (1 - t̄).
* §7.2: the sampler walks σ from 1 (noise) down to 0 (data) and applies the
  Euler update at each consecutive pair (σ, σ_next).
* §12.1: the recommended step count, guidance weight and shift per model and
  mode (for example 50 steps with shift 10 for audio-video, 4 steps with
  shift 5 for the robot policy).

Reading (the pages give the map, the step counts and the shifts, but not the
grid the sampler walks): an n-step schedule takes t = k/n, so
t̄_k = (n - k)/n, for k = 0..n, and maps each point through the shift.  That
gives σ_0 = 1 and σ_n = 0, the loop of §7.2, and for s = 1 the plain linear
schedule σ_k = 1 - k/n.

Everything is evaluated in float64, left to right as written above.
"""
from __future__ import annotations


def shift_sigma(t_bar: float, s: float) -> float:
    """σ = s·t̄ / (1 + (s - 1)·t̄) (§6.3)."""
    return s * t_bar / (1.0 + (s - 1.0) * t_bar)


def shifted_schedule(n_steps: int, shift: float):
    """σ_k for k = 0..n_steps on the uniform t grid, mapped through the
    shift.  Raises ValueError for n_steps < 1 or a shift that is not a
    positive finite number."""
    if n_steps < 1:
        raise ValueError("n_steps must be >= 1")
    if not (0.0 < shift < float("inf")):
        raise ValueError("shift must be positive and finite")
    return [shift_sigma(float(n_steps - k) / float(n_steps), float(shift)) for k in range(n_steps + 1)]
