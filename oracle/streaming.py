"""Streaming chunk generation against a rolling key/value cache.

News page "NVIDIA 发布 Cosmos 3 系列四个开放权重世界模型", section
"流式生成如何工作": the generator predicts each short chunk from the prompt,
the available controls and the generated history (control + history ->
generate chunk -> decode -> update history); temporal-causal attention reads
the history and hides future targets; a key/value cache keeps the attention
state for the next prediction; the distilled models take four denoising steps
per chunk and roll their history.

Readings (the page gives no cache policy):

* The key buffer is [AR prefix | ring of H history frame slots | current
  chunk].  The prefix is pinned; ring slot s holds the latest frame f with
  f mod H = s.  Cached keys are stored already rotated by mRoPE at their
  absolute positions, so slot order never matters to attention.
* During chunk c (absolute latent frame H + c) each denoising step attends
  the chunk's queries to the whole buffer under CHUNK_CAUSAL_KV (the chunk is
  the newest, so every cached key is visible; attention inside the chunk is
  full).  After the last step the chunk's rotated K and its V from that step
  overwrite slot c mod H.
"""
from __future__ import annotations

import numpy as np

from workloads import CHUNK_CAUSAL_KV
from . import attention, mrope


class RollingCache:
    def __init__(self, prefix_k, prefix_v, prefix_pos, hist_k, hist_v, hist_pos,
                 frame_tokens, sections, theta):
        """Raw (unrotated) keys are rotated here at their positions.
        hist_* hold ``slots`` frames back to back in slot order."""
        self.sections, self.theta = sections, theta
        self.ft = frame_tokens
        self.n_prefix = prefix_k.shape[0]
        self.slots = hist_k.shape[0] // frame_tokens
        self.k = np.concatenate([mrope.apply(prefix_k, prefix_pos, sections, theta),
                                 mrope.apply(hist_k, hist_pos, sections, theta)])
        self.v = np.concatenate([np.asarray(prefix_v, np.float64),
                                 np.asarray(hist_v, np.float64)])

    def attend(self, q_raw, k_raw, v_raw, pos, rows=None, heads=None):
        """One denoising step of the current chunk: returns O (all rows,
        or the selected rows x heads) and the chunk's rotated K."""
        qr = mrope.apply(q_raw, pos, self.sections, self.theta)
        kr = mrope.apply(k_raw, pos, self.sections, self.theta)
        kk = np.concatenate([self.k, kr])
        vv = np.concatenate([self.v, np.asarray(v_raw, np.float64)])
        q0 = self.k.shape[0]
        if rows is None:
            o, _ = attention.attention(qr, kk, vv, q0, CHUNK_CAUSAL_KV,
                                       n_prefix=self.n_prefix, chunk_len=self.ft)
        else:
            o = attention.attention_rows(qr[rows], kk, vv, rows, heads, q0,
                                         CHUNK_CAUSAL_KV, n_prefix=self.n_prefix,
                                         chunk_len=self.ft)
        return o, kr

    def append(self, chunk_index, k_rot, v_raw):
        s = chunk_index % self.slots
        a = self.n_prefix + s * self.ft
        self.k[a:a + self.ft] = k_rot
        self.v[a:a + self.ft] = np.asarray(v_raw, np.float64)
