"""Region-split projection ("Cosmos 3 方法原理全解" §3 and §3.2).

Each MoT layer holds two rooms with their own weights: AR tokens go through
the Reasoner's QKV (and output) projection, DM tokens through the
Generator's.  For a packed block of rows whose first ``n_ar`` rows are AR:

    Y[r] = X[r] @ W_ar   for r <  n_ar
    Y[r] = X[r] @ W_dm   for r >= n_ar

W is [d_in, d_out] row-major.  The fused QKV weight of a room is
[hidden, 3*H*D] with columns [Q | K | V], each laid out [H][D] (a reading of
the "3072x9216" weight shape; the pages give no layout).  The same map with
d_in = H*D and d_out = hidden is the output projection.
"""
from __future__ import annotations

import numpy as np


def project(x, w_ar, w_dm, n_ar: int) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    w_ar = np.asarray(w_ar, dtype=np.float64)
    w_dm = np.asarray(w_dm, dtype=np.float64)
    y = np.empty((x.shape[0], w_ar.shape[1]), dtype=np.float64)
    y[:n_ar] = x[:n_ar] @ w_ar
    y[n_ar:] = x[n_ar:] @ w_dm
    return y


def project_rows(x_rows, w, ) -> np.ndarray:
    """X[rows] @ W for a sample of rows that all lie in one region."""
    return np.asarray(x_rows, dtype=np.float64) @ np.asarray(w, dtype=np.float64)


def split_qkv(y: np.ndarray, n_heads: int, head_dim: int, n_kv_heads=None):
    """[N, (H + 2 H_kv) D] -> Q [N, H, D], K and V [N, H_kv, D] (columns
    [Q | K | V], each [heads][D]); H_kv defaults to H."""
    n = y.shape[0]
    hk = n_heads if n_kv_heads is None else n_kv_heads
    if y.shape[1] != (n_heads + 2 * hk) * head_dim:
        raise ValueError("QKV width is not (H + 2 H_kv) D")
    q = y[:, :n_heads * head_dim].reshape(n, n_heads, head_dim)
    k = y[:, n_heads * head_dim:(n_heads + hk) * head_dim].reshape(n, hk, head_dim)
    v = y[:, (n_heads + hk) * head_dim:].reshape(n, hk, head_dim)
    return q, k, v


def flops(n_rows: int, d_in: int, d_out: int) -> float:
    return 2.0 * n_rows * d_in * d_out
