"""Unified 3D mRoPE ("Cosmos 3 方法原理全解" §5).

Every token carries (t, h, w).  The head dimension D is split into P = D/2
rotary pairs; pair k rotates the two coordinates (x_k, x_{k+P}) (rotate-half
pairing) by the angle a = pos[axis(k)] * theta^(-2k/D).  The first s_t pairs
take t, the next s_h take h and the last s_w take w (s_t + s_h + s_w = P).

With t = h = w = p (text tokens) every pair sees the same p and the map is the
ordinary 1D RoPE, as §5 states; this is pinned by a test against an
independently written complex-number 1D RoPE.  Because the rotation of pair k
depends on the position only through a * pos, a uniform shift of all
positions leaves q_i . k_j unchanged (relative-position property).

Readings (the pages fix none of these): theta = 10000, rotate-half pairing,
one frequency ladder over all pairs, contiguous t|h|w sections.
"""
from __future__ import annotations

import numpy as np


def inv_freq(head_dim: int, theta: float) -> np.ndarray:
    k = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(theta) ** (-2.0 * k / head_dim)


def axis_of_pair(sections) -> np.ndarray:
    st, sh, sw = sections
    return np.array([0] * st + [1] * sh + [2] * sw, dtype=np.int64)


def angles(pos: np.ndarray, head_dim: int, sections, theta: float) -> np.ndarray:
    """[N, P] float64 rotation angles."""
    if sum(sections) * 2 != head_dim:
        raise ValueError("sections must cover D/2 pairs")
    p = np.asarray(pos, dtype=np.float64)
    return p[:, axis_of_pair(sections)] * inv_freq(head_dim, theta)[None, :]


def apply(x: np.ndarray, pos: np.ndarray, sections, theta: float) -> np.ndarray:
    """Rotate x [N, H, D] (any float) by its tokens' positions; float64 out."""
    x = np.asarray(x, dtype=np.float64)
    n, h, d = x.shape
    half = d // 2
    a = angles(pos, d, sections, theta)
    c = np.cos(a)[:, None, :]
    s = np.sin(a)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)
