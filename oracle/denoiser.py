"""One MoT layer of the denoiser forward, stripped to the joint-attention hot
path, chained into the sampler ("Cosmos 3 方法原理全解" §3 and §7.2-§7.3).

Per sampler step (sigma -> sigma_next):

    X   = [X_AR ; X_clean ; x]          rows of the packed sequence
    Y   = region-split QKV projection of X          (§3: two rooms)
    Q,K = mRoPE(Q, pos), mRoPE(K, pos)              (§5)
    O   = joint masked attention (AR causal, DM full)  (§3 equations)
    Z   = region-split output projection of O
    v   = the DM-noisy rows of Z
    x   = x + (sigma_next - sigma) * v              (§7.2)

Stripped on purpose: LayerNorm, MLP, residuals, CFG and the modality heads.
Reading: the noisy latent has ``hidden`` channels, so its rows enter X
directly (as bf16 in the bf16 workloads) and v is read from Z directly.

Parity of this chain is checked step by step with teacher forcing (each step
starts from the GPU's x); the free-running trajectory is parity unpinned
end to end: each stage is pinned on its own module, the composition is not.
"""
from __future__ import annotations

import numpy as np

from workloads import AR_CAUSAL_DM_FULL
from . import attention, euler, mrope, projection


def layer(X, w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm, pos, n_ar, n_heads, head_dim,
          sections, theta):
    """Returns dict of float64 intermediates: y, q, k, v, o, z."""
    n = X.shape[0]
    y = projection.project(X, w_qkv_ar, w_qkv_dm, n_ar)
    q, k, v = projection.split_qkv(y, n_heads, head_dim)
    qr = mrope.apply(q, pos, sections, theta)
    kr = mrope.apply(k, pos, sections, theta)
    o, lse = attention.attention(qr, kr, v, 0, AR_CAUSAL_DM_FULL, n_ar=n_ar)
    z = projection.project(o.reshape(n, n_heads * head_dim), w_o_ar, w_o_dm, n_ar)
    return dict(y=y, q=qr, k=kr, v=v, o=o, lse=lse, z=z)


def step(x, X_cond, w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm, pos, n_ar, n_heads,
         head_dim, sections, theta, sigma, sigma_next, x_as_input=None):
    """One sampler step.  ``X_cond`` holds the AR and clean rows; ``x`` the
    noisy latent (float32).  ``x_as_input`` is the value of x as it enters X
    (e.g. its bf16 rounding); defaults to x itself."""
    xin = x if x_as_input is None else x_as_input
    X = np.concatenate([np.asarray(X_cond, np.float64), np.asarray(xin, np.float64)], axis=0)
    inter = layer(X, w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm, pos, n_ar, n_heads,
                  head_dim, sections, theta)
    vel = inter["z"][X_cond.shape[0]:]
    inter["vel"] = vel
    inter["x_next"] = euler.step(x, vel, sigma, sigma_next)
    return inter
