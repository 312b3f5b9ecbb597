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

``store="bf16"`` is the same chain with bf16 activations: every tensor the
chain hands from one step of the path to the next is held in bfloat16, so
it is rounded (to nearest, ties to even, from the exact value) at those
points: the QKV output Y, the rotated Q and K, the attention output O and
the output projection Z.  Everything between those points stays float64.
The default ``store=None`` rounds nothing.

The composition is pinned on the CPU (tests/test_oracle_denoiser.py): an
independent build from explicit loops, the closed form with zero Q and K
weights, the relative-position invariance of the whole layer and the
permutation equivariance of the DM rows, each shown to catch planted
mistakes.
"""
from __future__ import annotations

import numpy as np

from workloads import AR_CAUSAL_DM_FULL
from . import attention, euler, mrope, projection


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits, ties
    to even), returned as float64.  Finite normal range only."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                  # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def layer(X, w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm, pos, n_ar, n_heads, head_dim,
          sections, theta, store=None, n_kv_heads=None):
    """Returns dict of float64 intermediates: y, q, k, v, o, lse, z.  With
    n_kv_heads, K and V have that many heads (grouped, oracle.attention)."""
    if store not in (None, "bf16"):
        raise ValueError("store is None or 'bf16'")
    keep = round_bf16 if store == "bf16" else (lambda t: t)
    n = X.shape[0]
    y = keep(projection.project(X, w_qkv_ar, w_qkv_dm, n_ar))
    q, k, v = projection.split_qkv(y, n_heads, head_dim, n_kv_heads)
    qr = keep(mrope.apply(q, pos, sections, theta))
    kr = keep(mrope.apply(k, pos, sections, theta))
    o, lse = attention.attention(qr, kr, v, 0, AR_CAUSAL_DM_FULL, n_ar=n_ar)
    o = keep(o)
    z = keep(projection.project(o.reshape(n, n_heads * head_dim), w_o_ar, w_o_dm, n_ar))
    return dict(y=y, q=qr, k=kr, v=v, o=o, lse=lse, z=z)


def step(x, X_cond, w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm, pos, n_ar, n_heads,
         head_dim, sections, theta, sigma, sigma_next, x_as_input=None, store=None):
    """One sampler step.  ``X_cond`` holds the AR and clean rows; ``x`` the
    noisy latent (float32).  ``x_as_input`` is the value of x as it enters X
    (e.g. its bf16 rounding); defaults to x itself."""
    xin = x if x_as_input is None else x_as_input
    X = np.concatenate([np.asarray(X_cond, np.float64), np.asarray(xin, np.float64)], axis=0)
    inter = layer(X, w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm, pos, n_ar, n_heads,
                  head_dim, sections, theta, store=store)
    vel = inter["z"][X_cond.shape[0]:]
    inter["vel"] = vel
    inter["x_next"] = euler.step(x, vel, sigma, sigma_next)
    return inter
