"""Orchestration of the hot path on one GPU: buffers and the order of the
C-ABI calls.  No arithmetic of the method happens here; every step runs in
libmotattn's kernels.

``DenoiserStep`` is one sampler step of one MoT layer stripped to the
joint-attention path ("Cosmos 3 方法原理全解" §3 and §7.2):

    Y = region-split QKV(X)             mot_qkv_project
    K = mRoPE(K)                        mrope_apply (in place, cached form)
    O = masked attention(Q, K, V)       mot_attention_fwd (Q rotated on load)
    Z = region-split O-projection(O)    mot_qkv_project
    x = x + (sigma_next - sigma) Z_noisy, and X_noisy = bf16(x)
                                        flow_euler_step

``StreamState`` is the rolling key/value cache of the streaming mode
("流式生成如何工作"): [AR prefix | ring of history frame slots | current
chunk], keys stored rotated.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _binding as B


def _dt(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class DenoiserStep:
    def __init__(self, wl, X, w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm, x_latent, device="cuda"):
        """X: [N, hidden] packed input rows (the noisy rows are overwritten
        from x_latent); weights [d_in, d_out]; x_latent fp32 [n_noisy, hidden].
        All tensors are moved to the device once."""
        self.wl = wl
        pos, reg, n_ar = B.mot_build_layout(wl.segments)
        self.n = pos.shape[0]
        self.n_ar = n_ar
        self.n_noisy = int((reg == 2).sum())
        self.r_noisy = self.n - self.n_noisy
        h, d, hid = wl.n_heads, wl.head_dim, wl.hidden
        dt = _dt(wl.dtype)
        self.pos = torch.from_numpy(pos).to(device)
        self.X = X.to(device=device, dtype=dt).contiguous()
        self.w = [t.to(device=device, dtype=dt).contiguous() for t in (w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm)]
        self.x = x_latent.to(device=device, dtype=torch.float32).contiguous()
        self.Y = torch.empty((self.n, 3 * h * d), dtype=dt, device=device)
        self.O = torch.empty((self.n, h * d), dtype=dt, device=device)
        self.Z = torch.empty((self.n, hid), dtype=dt, device=device)
        self.lse = None
        y4 = self.Y.view(self.n, 3, h, d)
        self.q, self.k, self.v = y4[:, 0], y4[:, 1], y4[:, 2]
        self.o3 = self.O.view(self.n, h, d)
        self.attn = B.attn_args(self.q, self.k, self.v, self.o3, mask=B.MOT_AR_CAUSAL_DM_FULL,
                                q0=0, n_ar=n_ar, q_pos=self.pos, sections=wl.sections,
                                theta=wl.theta)
        # the first step's packed input carries the starting latent
        self.X[self.r_noisy:].copy_(self.x.to(dt))

    def project_qkv(self):
        B.mot_qkv_project(self.X, self.w[0], self.w[1], self.Y, self.n_ar)

    def rope_k(self):
        B.mrope_apply(self.k, self.pos, self.wl.sections, self.wl.theta)

    def attention(self):
        B.mot_attention_fwd_args(self.attn)

    def project_o(self):
        B.mot_qkv_project(self.O, self.w[2], self.w[3], self.Z, self.n_ar)

    def euler(self, sigma, sigma_next):
        mirror = self.X[self.r_noisy:] if self.X.dtype == torch.bfloat16 else None
        B.flow_euler_step(self.x, self.Z[self.r_noisy:], sigma, sigma_next, x_bf16=mirror)
        if mirror is None:  # fp32 workloads: the next input is x itself
            self.X[self.r_noisy:].copy_(self.x)

    def step(self, sigma, sigma_next):
        self.project_qkv()
        self.rope_k()
        self.attention()
        self.project_o()
        self.euler(sigma, sigma_next)


class StreamState:
    """Rolling KV cache for chunk-causal streaming attention."""

    def __init__(self, n_heads, head_dim, n_prefix, frame_tokens, slots, sections, theta,
                 device="cuda"):
        self.h, self.d = n_heads, head_dim
        self.n_prefix, self.ft, self.slots = n_prefix, frame_tokens, slots
        self.sections, self.theta = sections, theta
        nk = n_prefix + (slots + 1) * frame_tokens
        self.nk = nk
        self.K = torch.empty((nk, n_heads, head_dim), dtype=torch.bfloat16, device=device)
        self.V = torch.empty_like(self.K)
        self.pos = torch.empty((nk, 3), dtype=torch.float32, device=device)
        self.q0 = n_prefix + slots * frame_tokens  # the current chunk's rows

    def fill(self, k_raw, v, pos):
        """Load prefix + history (raw keys, rotated here) into the cache."""
        n = k_raw.shape[0]
        self.K[:n].copy_(k_raw)
        self.V[:n].copy_(v)
        self.pos[:n].copy_(pos)
        B.mrope_apply(self.K[:n], self.pos[:n], self.sections, self.theta)

    def attend(self, q, k_raw, v, pos, out, lse=None):
        """One denoising step of the current chunk; q is rotated on load,
        the chunk's keys are rotated into the cache tail."""
        a = self.q0
        self.K[a:a + self.ft].copy_(k_raw)
        self.V[a:a + self.ft].copy_(v)
        self.pos[a:a + self.ft].copy_(pos)
        B.mrope_apply(self.K[a:a + self.ft], self.pos[a:a + self.ft], self.sections, self.theta)
        B.mot_attention_fwd(q, self.K, self.V, out, mask=B.MOT_CHUNK_CAUSAL_KV, q0=self.q0,
                            n_prefix=self.n_prefix, chunk_len=self.ft, q_pos=pos,
                            sections=self.sections, theta=self.theta, lse=lse)

    def append(self, chunk_index):
        """Move the current chunk (rotated K, V, positions) into its ring slot."""
        s = chunk_index % self.slots
        dst = self.n_prefix + s * self.ft
        a = self.q0
        self.K[dst:dst + self.ft].copy_(self.K[a:a + self.ft])
        self.V[dst:dst + self.ft].copy_(self.V[a:a + self.ft])
        self.pos[dst:dst + self.ft].copy_(self.pos[a:a + self.ft])
