"""Masked softmax attention over the packed MoT sequence.

The joint-attention equations of "Cosmos 3 方法原理全解" §3 (O_AR causal over
the AR tokens, O_DM full over [K_AR; K_DM]) and the chunk-causal streaming
attention of "流式生成如何工作" are one computation under two masks (see
``oracle.mask``): for each head,

    S = Q K^T * scale,  S[i, j] = -inf where (i, j) is not allowed,
    P = row-softmax(S) (the row maximum is subtracted first),
    O = P V,            LSE_i = m_i + log sum_j exp(S_ij - m_i).

Reading: the pages write a bare Attn(.), so scale = 1/sqrt(D).

Grouped keys and values (the model table of the method page, §12.4, lists
Q / KV heads 16 / 8, 32 / 8 and 64 / 8): K and V may carry H_kv heads for
H query heads, H_kv dividing H; query head h reads key/value head
h // (H / H_kv).  With H_kv = H this is ordinary multi-head attention.

``attention`` is the vectorised definition, evaluated in float64 per head
on blocks of query rows (rows are independent, so blocking changes nothing).
``attention_rows`` evaluates the same definition for a chosen subset of
(query, head) outputs, which is what the full-size checks use.
``attention_bruteforce`` is the same definition written as explicit loops,
used only to pin the vectorised version on tiny inputs.
"""
from __future__ import annotations

import math

import numpy as np

from . import mask as _mask


def kv_head(h: int, n_heads: int, n_kv_heads: int) -> int:
    """Key/value head read by query head h (grouped heads, §12.4)."""
    if n_kv_heads < 1 or n_heads % n_kv_heads:
        raise ValueError("n_kv_heads must divide n_heads")
    return h // (n_heads // n_kv_heads)


def attention(q, k, v, q0, mode, n_ar=0, n_prefix=0, chunk_len=1, scale=None,
              row_block=256):
    """q [nq,H,D], k/v [nk,H_kv,D] -> (O [nq,H,D] float64, LSE [H,nq] float64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nh, d = q.shape
    nk, nkv = k.shape[0], k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.empty((nq, nh, d), dtype=np.float64)
    lse = np.empty((nh, nq), dtype=np.float64)
    for r0 in range(0, nq, row_block):
        r1 = min(nq, r0 + row_block)
        m = _mask.materialize(r1 - r0, nk, q0 + r0, mode, n_ar, n_prefix, chunk_len)
        # keys beyond the last allowed one never contribute; trimming them is
        # an exact saving for the causal AR rows
        kmax = int(np.nonzero(m.any(axis=0))[0].max()) + 1
        m = m[:, :kmax]
        for h in range(nh):
            g = kv_head(h, nh, nkv)
            s = (q[r0:r1, h, :] @ k[:kmax, g, :].T) * scale
            s = np.where(m, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            p = np.exp(s - mx)
            den = p.sum(axis=1, keepdims=True)
            o[r0:r1, h, :] = (p @ v[:kmax, g, :]) / den
            lse[h, r0:r1] = mx[:, 0] + np.log(den[:, 0])
    return o, lse


def attention_rows(q_rows, k, v, rows, heads, q0, mode, n_ar=0, n_prefix=0,
                   chunk_len=1, scale=None, kv_heads=None):
    """Outputs for selected (row, head) pairs.

    q_rows [len(rows), H, D] holds the query vectors of ``rows`` (indices
    into the query block); returns O [len(rows), len(heads), D] float64.
    ``heads`` index the query heads of q_rows; with ``kv_heads`` given, k / v
    carry only those key/value heads and kv_heads[b] is the index into them
    that heads[b] reads (default: the same index, H_kv = H).
    Rows whose allowed key sets are identical are evaluated together (the
    same definition, one matrix product per group).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    d = q_rows.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nk = k.shape[0]
    out = np.empty((len(rows), len(heads), d), dtype=np.float64)
    j = np.arange(nk, dtype=np.int64)
    groups = {}
    for a, r in enumerate(rows):
        allow = _mask.allowed(q0 + int(r), j, mode, n_ar, n_prefix, chunk_len)
        idx = np.nonzero(allow)[0]
        key = ("prefix", len(idx)) if idx[-1] + 1 == len(idx) else ("row", a)
        groups.setdefault(key, (idx, []))[1].append(a)
    for b, h in enumerate(heads):
        g = h if kv_heads is None else kv_heads[b]
        kh = np.asarray(k[:, g, :], dtype=np.float64)
        vh = np.asarray(v[:, g, :], dtype=np.float64)
        for key, (idx, members) in groups.items():
            kk = kh[:len(idx)] if key[0] == "prefix" else kh[idx]
            vv = vh[:len(idx)] if key[0] == "prefix" else vh[idx]
            s = (q_rows[members, h, :] @ kk.T) * scale
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[members, b, :] = (p @ vv) / p.sum(axis=1, keepdims=True)
    return out


def attention_bruteforce(q, k, v, q0, mode, n_ar=0, n_prefix=0, chunk_len=1,
                         scale=None):
    """Explicit-loop evaluation of the definition (tiny inputs only)."""
    nq, nh, d = len(q), len(q[0]), len(q[0][0])
    nk, nkv = len(k), len(k[0])
    group = nh // nkv  # query heads per key/value head
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = [[[0.0] * d for _ in range(nh)] for _ in range(nq)]
    lse = [[0.0] * nq for _ in range(nh)]
    for r in range(nq):
        i = q0 + r
        keys = [j for j in range(nk)
                if bool(_mask.allowed(i, j, mode, n_ar, n_prefix, chunk_len))]
        for h in range(nh):
            g = h // group
            scores = []
            for j in keys:
                acc = 0.0
                for e in range(d):
                    acc += float(q[r][h][e]) * float(k[j][g][e])
                scores.append(acc * scale)
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = sum(w)
            for e in range(d):
                acc = 0.0
                for wj, j in zip(w, keys):
                    acc += wj * float(v[j][g][e])
                o[r][h][e] = acc / tot
            lse[h][r] = mx + math.log(tot)
    return np.array(o), np.array(lse)


def merge(o_parts, lse_parts):
    """Combine attention over disjoint key sets into attention over their
    union: with L = log sum_b exp(L_b), O = sum_b exp(L_b - L) O_b and the
    union's LSE is L.  o_parts [B, nq, H, D], lse_parts [B, H, nq]; a part
    with no keys for a row has L_b = -inf and weight 0."""
    o = np.asarray(o_parts, dtype=np.float64)
    l = np.asarray(lse_parts, dtype=np.float64)
    m = l.max(axis=0)
    w = np.exp(l - m[None])                    # [B, H, nq]
    tot = w.sum(axis=0)
    lse = m + np.log(tot)
    wt = np.transpose(w / tot[None], (0, 2, 1))[..., None]  # [B, nq, H, 1]
    return (wt * o).sum(axis=0), lse


def flops(pairs: int, n_heads: int, head_dim: int) -> float:
    """Algorithmic FLOPs of masked attention: 2*D for q.k and 2*D for p*v
    per allowed (query, key, head) triple; masked pairs are not counted."""
    return 4.0 * head_dim * n_heads * pairs
