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

``GuidedDenoiserStep`` is a classifier-free-guided sampler step of the same
layer (§7.2 CFG equation, §7.3 generation loop): the condition and baseline
prompts' AR keys and values are computed once per request, and each step
runs the DM rows only, both predictions in one attention launch, and one
guided Euler pass.

``BlockStep`` is the whole MoT layer (§3: each room has its own LayerNorm,
QKV, output projection and MLP) over the packed rows:

    U1 = LN1(X)                         mot_layernorm_region
    Y  = QKV(U1); K = mRoPE(K)          mot_qkv_project, mrope_apply
    O  = attention                      mot_attention_fwd (Q rotated on load)
    H1 = X + Oproj(O)                   mot_region_linear (residual add)
    U2 = LN2(H1)                        mot_layernorm_region
    A  = GELU(U2 W_up)                  mot_region_linear (GELU)
    H2 = H1 + A W_down                  mot_region_linear (residual add)

``sample`` is the generation loop (§7.3) over a flow-shifted noise
schedule (§6.3 shift map; §12.1 recommended steps and shift per mode): the
noise levels come from mot_sigma_schedule and each consecutive pair drives
one step of a DenoiserStep or GuidedDenoiserStep.

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
        hk = getattr(wl, "n_kv_heads", 0) or h
        dt = _dt(wl.dtype)
        self.pos = torch.from_numpy(pos).to(device)
        self.X = X.to(device=device, dtype=dt).contiguous()
        self.w = [t.to(device=device, dtype=dt).contiguous() for t in (w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm)]
        self.x = x_latent.to(device=device, dtype=torch.float32).contiguous()
        self.Y = torch.empty((self.n, (h + 2 * hk) * d), dtype=dt, device=device)
        self.O = torch.empty((self.n, h * d), dtype=dt, device=device)
        self.Z = torch.empty((self.n, hid), dtype=dt, device=device)
        self.lse = None
        # columns [Q (H heads) | K (H_kv) | V (H_kv)], each [heads][D]
        self.q = self.Y[:, :h * d].view(self.n, h, d)
        self.k = self.Y[:, h * d:(h + hk) * d].view(self.n, hk, d)
        self.v = self.Y[:, (h + hk) * d:].view(self.n, hk, d)
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


class GuidedDenoiserStep:
    """Guided sampler step of the one-layer chain.

    Reading: the baseline prompt takes as many AR rows as the condition
    prompt, so the DM tokens keep their positions and, in one layer, their
    queries, keys and values are the same in both predictions.  Every DM
    query reads every key, so the order of its keys does not matter, and one
    packed QKV buffer holds both predictions' keys without copies:

        rows [0, n_ar)                the condition prompt's AR rows
        rows [n_ar, n_ar + n_dm)      the DM rows of the current step
        rows [n_ar + n_dm, N + n_ar)  the baseline prompt's AR rows

    The condition prediction reads keys [0, N), the baseline prediction
    keys [n_ar, n_ar + N); both share the DM queries.  O and Z hold the two
    predictions' DM rows ([2, n_dm, ...]); v_cond and v_base are their noisy
    rows.
    """

    def __init__(self, wl, X_ar_cond, X_ar_base, X_clean, w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm,
                 x_latent, guidance, device="cuda"):
        self.wl = wl
        pos, reg, n_ar = B.mot_build_layout(wl.segments)
        self.n = pos.shape[0]
        self.n_ar = n_ar
        self.n_dm = self.n - n_ar
        self.n_noisy = int((reg == 2).sum())
        self.n_clean = self.n_dm - self.n_noisy
        self.guidance = float(guidance)
        h, d, hid = wl.n_heads, wl.head_dim, wl.hidden
        hk = getattr(wl, "n_kv_heads", 0) or h
        dt = _dt(wl.dtype)
        width = (h + 2 * hk) * d
        self.pos = torch.from_numpy(pos).to(device)
        self.pos_dm = self.pos[n_ar:]
        self.w = [t.to(device=device, dtype=dt).contiguous() for t in (w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm)]
        self.x = x_latent.to(device=device, dtype=torch.float32).contiguous()
        rows = self.n + n_ar
        self.QKV = torch.empty((rows, width), dtype=dt, device=device)
        self.Xdm = torch.empty((self.n_dm, hid), dtype=dt, device=device)
        self.Xdm[:self.n_clean].copy_(X_clean.to(device=device, dtype=dt))
        self.Xdm[self.n_clean:].copy_(self.x.to(dt))
        self.O = torch.empty((2, self.n_dm, h * d), dtype=dt, device=device)
        self.Z = torch.empty((2, self.n_dm, hid), dtype=dt, device=device)
        # per request: both prompts' AR rows through the Reasoner weights,
        # keys rotated at the AR positions
        a_cond = self.QKV[:n_ar]
        a_base = self.QKV[n_ar + self.n_dm:]
        for X_ar, dst in ((X_ar_cond, a_cond), (X_ar_base, a_base)):
            if n_ar == 0:
                break
            B.mot_qkv_project(X_ar.to(device=device, dtype=dt).contiguous(), self.w[0], None, dst, n_ar)
            B.mrope_apply(dst[:, h * d:(h + hk) * d].view(n_ar, hk, d), self.pos[:n_ar],
                          wl.sections, wl.theta)
        # views of the per-step buffers
        dm = self.QKV[n_ar:n_ar + self.n_dm]
        self.Ydm = dm
        self.k_dm = dm[:, h * d:(h + hk) * d].view(self.n_dm, hk, d)
        st = self.QKV.stride(0)
        base = self.QKV.storage_offset()
        q = dm[:, :h * d].view(self.n_dm, h, d).unsqueeze(0).expand(2, self.n_dm, h, d)
        k = torch.as_strided(self.QKV, (2, self.n, hk, d), (n_ar * st, st, d, 1), base + h * d)
        v = torch.as_strided(self.QKV, (2, self.n, hk, d), (n_ar * st, st, d, 1), base + (h + hk) * d)
        o = self.O.view(2, self.n_dm, h, d)
        # every query is a DM row (q0 = n_ar), so every key is allowed
        self.attn = B.attn_args(q, k, v, o, mask=B.MOT_AR_CAUSAL_DM_FULL, q0=n_ar, n_ar=n_ar,
                                q_pos=self.pos_dm, sections=wl.sections, theta=wl.theta)

    def project_qkv(self):
        B.mot_qkv_project(self.Xdm, None, self.w[1], self.Ydm, 0)

    def rope_k(self):
        B.mrope_apply(self.k_dm, self.pos_dm, self.wl.sections, self.wl.theta)

    def attention(self):
        B.mot_attention_fwd_args(self.attn)

    def project_o(self):
        B.mot_qkv_project(self.O.view(2 * self.n_dm, -1), None, self.w[3],
                          self.Z.view(2 * self.n_dm, -1), 0)

    def euler(self, sigma, sigma_next):
        c = self.n_clean
        mirror = self.Xdm[c:] if self.Xdm.dtype == torch.bfloat16 else None
        B.flow_cfg_euler_step(self.x, self.Z[0, c:], self.Z[1, c:], self.guidance, sigma, sigma_next,
                              x_bf16=mirror)
        if mirror is None:
            self.Xdm[c:].copy_(self.x)

    def step(self, sigma, sigma_next):
        self.project_qkv()
        self.rope_k()
        self.attention()
        self.project_o()
        self.euler(sigma, sigma_next)


def sample(stepper, n_steps, shift):
    """Runs ``stepper.step(sigma_k, sigma_{k+1})`` for k = 0 .. n_steps - 1
    over the schedule sigma_0 = 1 .. sigma_n = 0 that mot_sigma_schedule
    builds for ``shift`` (shift 1 is the linear schedule).  ``stepper`` is a
    DenoiserStep or GuidedDenoiserStep; its latent ends at sigma = 0.
    Returns the float32 schedule that was used."""
    sig = B.mot_sigma_schedule(n_steps, shift)
    for k in range(int(n_steps)):
        stepper.step(float(sig[k]), float(sig[k + 1]))
    return sig


class BlockStep:
    """The whole MoT layer's forward over one packed block of rows."""

    def __init__(self, wl, X, params, device="cuda", eps=1e-6):
        """X: [N, hidden] packed rows; params: ln1_ar, ln1_dm, ln2_ar, ln2_dm
        ((gamma, beta) pairs of fp32 tensors) and qkv_ar, qkv_dm, o_ar, o_dm,
        up_ar, up_dm, down_ar, down_dm (matrices [d_in, d_out])."""
        self.wl = wl
        pos, reg, n_ar = B.mot_build_layout(wl.segments)
        self.n, self.n_ar, self.eps = pos.shape[0], n_ar, eps
        h, d, hid, ffn = wl.n_heads, wl.head_dim, wl.hidden, wl.ffn
        hk = getattr(wl, "n_kv_heads", 0) or h
        dt = _dt(wl.dtype)
        n = self.n
        dev = lambda t, ty: t.to(device=device, dtype=ty).contiguous()
        self.p = {}
        for k, v in params.items():
            self.p[k] = tuple(dev(t, torch.float32) for t in v) if k.startswith("ln") else dev(v, dt)
        self.pos = torch.from_numpy(pos).to(device)
        self.X = dev(X, dt)
        self.U = torch.empty((n, hid), dtype=dt, device=device)
        self.Y = torch.empty((n, (h + 2 * hk) * d), dtype=dt, device=device)
        self.O = torch.empty((n, h * d), dtype=dt, device=device)
        self.H1 = torch.empty((n, hid), dtype=dt, device=device)
        self.A = torch.empty((n, ffn), dtype=dt, device=device)
        self.H2 = torch.empty((n, hid), dtype=dt, device=device)
        self.q = self.Y[:, :h * d].view(n, h, d)
        self.k = self.Y[:, h * d:(h + hk) * d].view(n, hk, d)
        self.v = self.Y[:, (h + hk) * d:].view(n, hk, d)
        self.attn = B.attn_args(self.q, self.k, self.v, self.O.view(n, h, d),
                                mask=B.MOT_AR_CAUSAL_DM_FULL, q0=0, n_ar=n_ar, q_pos=self.pos,
                                sections=wl.sections, theta=wl.theta)

    def ln1(self):
        B.mot_layernorm_region(self.X, self.U, self.n_ar, self.p["ln1_ar"], self.p["ln1_dm"], self.eps)

    def project_qkv(self):
        B.mot_qkv_project(self.U, self.p["qkv_ar"], self.p["qkv_dm"], self.Y, self.n_ar)

    def rope_k(self):
        B.mrope_apply(self.k, self.pos, self.wl.sections, self.wl.theta)

    def attention(self):
        B.mot_attention_fwd_args(self.attn)

    def project_o(self):
        B.mot_region_linear(self.O, self.p["o_ar"], self.p["o_dm"], self.H1, self.n_ar,
                            B.MOT_EPI_ADD, residual=self.X)

    def ln2(self):
        B.mot_layernorm_region(self.H1, self.U, self.n_ar, self.p["ln2_ar"], self.p["ln2_dm"], self.eps)

    def mlp_up(self):
        B.mot_region_linear(self.U, self.p["up_ar"], self.p["up_dm"], self.A, self.n_ar, B.MOT_EPI_GELU)

    def mlp_down(self):
        B.mot_region_linear(self.A, self.p["down_ar"], self.p["down_dm"], self.H2, self.n_ar,
                            B.MOT_EPI_ADD, residual=self.H1)

    def forward(self):
        for f in (self.ln1, self.project_qkv, self.rope_k, self.attention, self.project_o,
                  self.ln2, self.mlp_up, self.mlp_down):
            f()


class StreamState:
    """Rolling KV cache for chunk-causal streaming attention.

    With split = 2 each call splits its keys in two halves over a batch of
    two launches (item b reads keys [b nk/2, (b+1) nk/2); the newest chunk
    sees every key, so each half is plain full attention) and merges the
    halves' outputs through their LSE: twice the workgroups for the same
    query tiles."""

    def __init__(self, n_heads, head_dim, n_prefix, frame_tokens, slots, sections, theta,
                 device="cuda", split=1):
        self.h, self.d = n_heads, head_dim
        self.n_prefix, self.ft, self.slots = n_prefix, frame_tokens, slots
        self.sections, self.theta = sections, theta
        nk = n_prefix + (slots + 1) * frame_tokens
        self.nk = nk
        self.K = torch.empty((nk, n_heads, head_dim), dtype=torch.bfloat16, device=device)
        self.V = torch.empty_like(self.K)
        self.pos = torch.empty((nk, 3), dtype=torch.float32, device=device)
        self.q0 = n_prefix + slots * frame_tokens  # the current chunk's rows
        if split not in (1, 2) or (split == 2 and nk % 2):
            raise ValueError("split is 1, or 2 with an even key count")
        self.split = split
        if split == 2:
            self.O_parts = torch.empty((2, frame_tokens, n_heads, head_dim), dtype=torch.bfloat16,
                                       device=device)
            self.L_parts = torch.empty((2, n_heads, frame_tokens), dtype=torch.float32, device=device)

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
        if self.split == 1:
            B.mot_attention_fwd(q, self.K, self.V, out, mask=B.MOT_CHUNK_CAUSAL_KV, q0=self.q0,
                                n_prefix=self.n_prefix, chunk_len=self.ft, q_pos=pos,
                                sections=self.sections, theta=self.theta, lse=lse)
            return
        # the chunk is the newest: every key is visible, so each half of the
        # keys is full attention (every query row a DM row of the AR mask)
        half = self.nk // 2
        k2 = torch.as_strided(self.K, (2, half, self.h, self.d),
                              (half * self.K.stride(0),) + tuple(self.K.stride()), self.K.storage_offset())
        v2 = torch.as_strided(self.V, (2, half, self.h, self.d),
                              (half * self.V.stride(0),) + tuple(self.V.stride()), self.V.storage_offset())
        q2 = q.unsqueeze(0).expand(2, *q.shape)
        B.mot_attention_fwd(q2, k2, v2, self.O_parts, mask=B.MOT_AR_CAUSAL_DM_FULL, q0=0, n_ar=0,
                            q_pos=pos, sections=self.sections, theta=self.theta, lse=self.L_parts)
        B.mot_attention_merge(self.O_parts, self.L_parts, out, lse=lse)

    def append(self, chunk_index):
        """Move the current chunk (rotated K, V, positions) into its ring slot."""
        s = chunk_index % self.slots
        dst = self.n_prefix + s * self.ft
        a = self.q0
        self.K[dst:dst + self.ft].copy_(self.K[a:a + self.ft])
        self.V[dst:dst + self.ft].copy_(self.V[a:a + self.ft])
        self.pos[dst:dst + self.ft].copy_(self.pos[a:a + self.ft])
