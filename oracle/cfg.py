"""Classifier-free guidance in the sampler ("Cosmos 3 方法原理全解" §7.2,
the CFG equation, and §7.3, the generation loop).

The Reasoner encodes the condition prompt and the baseline prompt (empty or
negative) once per request; their AR keys and values are cached.  Every
sampler step then makes two Generator predictions on the same DM block
(clean conditions followed by the current latent): v_cond reads the
condition prompt's cached AR keys and values, v_base the baseline's.  The
step combines them,

    v = v_base + w (v_cond - v_base),

and takes the Euler update x_next = x + (sigma_next - sigma) v (§7.2).

Readings (the pages leave these open):

* The baseline prompt occupies as many AR tokens as the condition prompt
  (the request pads it), so both branches lay out the packed sequence alike
  and every DM token keeps its position.  In the one-layer chain the DM
  rows' queries, keys and values are then the same in both branches; only
  the AR keys and values differ.
* The guidance weight w is a float32, like the sigmas handed to the kernel.
"""
from __future__ import annotations

import numpy as np

from . import denoiser, euler


def combine(v_cond, v_base, w: float) -> np.ndarray:
    """v_base + w (v_cond - v_base), in float64 (§7.2)."""
    wf = np.float64(np.float32(w))
    vb = np.asarray(v_base, dtype=np.float64)
    return vb + wf * (np.asarray(v_cond, dtype=np.float64) - vb)


def euler_step(x, v_cond, v_base, w: float, sigma: float, sigma_next: float) -> np.ndarray:
    """The sampler update with the guided velocity."""
    return euler.step(x, combine(v_cond, v_base, w), sigma, sigma_next)


def step(x, X_ar_cond, X_ar_base, X_clean, w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm, pos, n_ar,
         n_heads, head_dim, sections, theta, w, sigma, sigma_next, x_as_input=None, store=None,
         n_kv_heads=None):
    """One guided sampler step of the one-layer chain: the two Generator
    predictions are each the full packed-sequence layer of
    ``oracle.denoiser`` with that branch's AR rows, and v is read from the
    DM-noisy rows.  Returns the two velocities, the guided one and x_next."""
    if np.shape(X_ar_cond) != np.shape(X_ar_base):
        raise ValueError("the baseline prompt takes as many AR rows as the condition prompt")
    xin = x if x_as_input is None else x_as_input
    out = {}
    for name, X_ar in (("cond", X_ar_cond), ("base", X_ar_base)):
        X = np.concatenate([np.asarray(X_ar, np.float64), np.asarray(X_clean, np.float64).reshape(
            -1, np.shape(X_ar)[1]), np.asarray(xin, np.float64)], axis=0)
        inter = denoiser.layer(X, w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm, pos, n_ar, n_heads, head_dim,
                               sections, theta, store=store, n_kv_heads=n_kv_heads)
        out["vel_" + name] = inter["z"][X.shape[0] - np.shape(xin)[0]:]
    out["vel"] = combine(out["vel_cond"], out["vel_base"], w)
    out["x_next"] = euler.step(x, out["vel"], sigma, sigma_next)
    return out
