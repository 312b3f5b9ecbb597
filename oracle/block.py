"""The whole MoT layer ("Cosmos 3 方法原理全解" §3, §3.2): each room (the
Reasoner for AR tokens, the Generator for DM tokens) has its own LayerNorm,
QKV projection, output projection and MLP; the joint attention of §3 is the
only place the rooms meet.  §12.4's model table gives the MLP width (FFN)
per model.

For the packed rows X [N, hidden] whose first n_ar rows are AR:

    H1 = X  + Oproj(Attn(mRoPE(QKV(LN1(X)))))      (oracle.denoiser's path)
    H2 = H1 + MLP(LN2(H1)),   MLP(u) = GELU(u W_up) W_down

with every LayerNorm, projection and MLP matrix taken from the row's room.

Readings (the pages name the parts but not their form):

* LayerNorm is the standard one over the hidden dimension,
  (x - mean) / sqrt(var + eps) * gamma + beta, with the biased variance and
  eps = 1e-6, and its own gamma and beta per room.
* The MLP has two matrices, hidden -> FFN -> hidden, no biases, and GELU in
  its exact form x Phi(x) = x (1 + erf(x / sqrt 2)) / 2 between them.
* The layer is pre-norm with residual connections around the attention and
  the MLP, the plainest transformer layer the pages' "LayerNorm, QKV and
  MLP" describes.

``store="bf16"`` rounds to bfloat16 where the bf16 path stores a tensor:
LN outputs, the QKV output, rotated Q and K, the attention output, H1, the
activated MLP hidden layer and H2.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

from workloads import AR_CAUSAL_DM_FULL
from . import attention, denoiser, mrope, projection

EPS = 1e-6


def layer_norm(x, gamma, beta, eps: float = EPS) -> np.ndarray:
    """Row-wise LayerNorm of x [N, C] with gamma, beta [C]."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def region_layer_norm(x, ln_ar, ln_dm, n_ar: int, eps: float = EPS) -> np.ndarray:
    """LayerNorm with the Reasoner's (gamma, beta) on rows < n_ar and the
    Generator's on the rest."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    out[:n_ar] = layer_norm(x[:n_ar], *ln_ar, eps)
    out[n_ar:] = layer_norm(x[n_ar:], *ln_dm, eps)
    return out


def gelu(x) -> np.ndarray:
    """x Phi(x), Phi the standard normal CDF, via erf."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def mlp(u, w_up_ar, w_up_dm, w_down_ar, w_down_dm, n_ar: int, store=None) -> np.ndarray:
    keep = denoiser.round_bf16 if store == "bf16" else (lambda t: t)
    a = keep(gelu(projection.project(u, w_up_ar, w_up_dm, n_ar)))
    return projection.project(a, w_down_ar, w_down_dm, n_ar)


def layer(X, p, pos, n_ar, n_heads, head_dim, sections, theta, store=None, n_kv_heads=None,
          eps: float = EPS):
    """One MoT layer.  ``p`` maps names to arrays: ln1_ar, ln1_dm, ln2_ar,
    ln2_dm (each a (gamma, beta) pair), qkv_ar, qkv_dm, o_ar, o_dm, up_ar,
    up_dm, down_ar, down_dm.  Returns float64 intermediates including h1 and
    the output h2."""
    keep = denoiser.round_bf16 if store == "bf16" else (lambda t: t)
    X = np.asarray(X, dtype=np.float64)
    n = X.shape[0]
    u1 = keep(region_layer_norm(X, p["ln1_ar"], p["ln1_dm"], n_ar, eps))
    y = keep(projection.project(u1, p["qkv_ar"], p["qkv_dm"], n_ar))
    q, k, v = projection.split_qkv(y, n_heads, head_dim, n_kv_heads)
    qr = keep(mrope.apply(q, pos, sections, theta))
    kr = keep(mrope.apply(k, pos, sections, theta))
    o, _ = attention.attention(qr, kr, v, 0, AR_CAUSAL_DM_FULL, n_ar=n_ar)
    o = keep(o)
    h1 = keep(X + projection.project(o.reshape(n, n_heads * head_dim), p["o_ar"], p["o_dm"], n_ar))
    u2 = keep(region_layer_norm(h1, p["ln2_ar"], p["ln2_dm"], n_ar, eps))
    h2 = keep(h1 + mlp(u2, p["up_ar"], p["up_dm"], p["down_ar"], p["down_dm"], n_ar, store))
    return dict(u1=u1, y=y, q=qr, k=kr, v=v, o=o, h1=h1, u2=u2, h2=h2)
