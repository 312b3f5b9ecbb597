"""Attention masks of the packed sequence, and tile classes.

AR_CAUSAL_DM_FULL follows "Cosmos 3 方法原理全解" §3: O_AR is causal
attention over the AR tokens only (the Reasoner stays a valid autoregressive
model and never reads DM), and O_DM is full attention of every DM query over
[K_AR; K_DM] (all text and all DM tokens, bidirectional inside DM).  In the
absolute index space of the packed sequence, query i may read key j iff
``i >= n_ar`` or ``j <= i``.

CHUNK_CAUSAL_KV follows the news page on the four new Cosmos 3 checkpoints,
section "流式生成如何工作": temporal-causal attention reads the available
history and controls and hides future targets, with a key/value cache kept
for the next prediction.  Keys [0, n_prefix) are the cached AR prefix and are
visible to every query; past it, keys are grouped into chunks of
``chunk_len`` and query i may read key j iff chunk(j) <= chunk(i), with
chunk(x) = floor((x - n_prefix) / chunk_len).  Attention inside a chunk is
full.

Query row r has absolute index i = q0 + r in the key space.
"""
from __future__ import annotations

import numpy as np

from workloads import AR_CAUSAL_DM_FULL, CHUNK_CAUSAL_KV

EMPTY, PARTIAL, FULL = 0, 1, 2


def allowed(i, j, mode, n_ar=0, n_prefix=0, chunk_len=1):
    """Vectorised predicate over broadcastable absolute indices i, j."""
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    if mode == AR_CAUSAL_DM_FULL:
        return (i >= n_ar) | (j <= i)
    if mode == CHUNK_CAUSAL_KV:
        cj = np.floor_divide(j - n_prefix, chunk_len)
        ci = np.floor_divide(i - n_prefix, chunk_len)
        return (j < n_prefix) | (cj <= ci)
    raise ValueError("unknown mask mode")


def materialize(nq, nk, q0, mode, n_ar=0, n_prefix=0, chunk_len=1):
    """Boolean [nq, nk] mask."""
    i = (q0 + np.arange(nq, dtype=np.int64))[:, None]
    j = np.arange(nk, dtype=np.int64)[None, :]
    return allowed(i, j, mode, n_ar, n_prefix, chunk_len)


def tile_classes(m: np.ndarray, bm: int, bn: int) -> np.ndarray:
    """EMPTY / PARTIAL / FULL per (bm x bn) tile of a boolean mask; a ragged
    edge tile is judged on its in-range pairs only."""
    nq, nk = m.shape
    tq, tk = -(-nq // bm), -(-nk // bn)
    out = np.empty((tq, tk), dtype=np.uint8)
    for a in range(tq):
        for b in range(tk):
            blk = m[a * bm:(a + 1) * bm, b * bn:(b + 1) * bn]
            if not blk.any():
                out[a, b] = EMPTY
            elif blk.all():
                out[a, b] = FULL
            else:
                out[a, b] = PARTIAL
    return out


def count_pairs(nq, nk, q0, mode, n_ar=0, n_prefix=0, chunk_len=1, block=4096):
    """Number of allowed (query, key) pairs, by rows in blocks."""
    total = 0
    for r0 in range(0, nq, block):
        r1 = min(nq, r0 + block)
        total += int(materialize(r1 - r0, nk, q0 + r0, mode, n_ar, n_prefix,
                                 chunk_len).sum())
    return total
