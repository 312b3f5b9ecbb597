"""Seeded synthetic workloads for the MoT joint-attention hot path.

This module is shared by the tests, the benchmark and the CPU oracle checks.
It holds *data only*: the five workload descriptions (segment lists, head
shapes, dtypes, sigma schedules) and counter-free seeded random generators.
It contains none of the method's arithmetic: token positions, masks, rotary
angles, attention, projections and the sampler update are computed
independently by the oracle and by the HIP library.

Every random tensor is drawn from ``numpy.random.default_rng([workload_id,
tensor_id])`` (PCG64), so any tensor can be regenerated alone and in any order.
Activations are N(0,1), weights N(0, 0.02); bf16 workloads round the fp32
draw to bfloat16 with round-to-nearest-even, and both sides read those bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

# Region tags (the clean/noisy task switch of the packed sequence).
AR, DM_CLEAN, DM_NOISY = 0, 1, 2
REGION_NAMES = {AR: "AR", DM_CLEAN: "DM_CLEAN", DM_NOISY: "DM_NOISY"}

# Token kinds inside a region.
TEXT, SPECIAL, VIDEO, AUDIO, ACTION, PROPRIO = 0, 1, 2, 3, 4, 5
KIND_NAMES = {TEXT: "TEXT", SPECIAL: "SPECIAL", VIDEO: "VIDEO", AUDIO: "AUDIO",
              ACTION: "ACTION", PROPRIO: "PROPRIO"}

# Mask modes.
AR_CAUSAL_DM_FULL, CHUNK_CAUSAL_KV = 0, 1


@dataclass(frozen=True)
class Segment:
    """One group of tokens in the packed sequence.

    ``n_tokens`` counts TEXT / SPECIAL / AUDIO / ACTION / PROPRIO tokens.
    VIDEO groups give ``n_frames`` latent frames of ``n_views`` camera views on
    a ``grid_h`` x ``grid_w`` latent grid.  ``rate`` is the token rate on the
    time axis: tokens per second for AUDIO / ACTION, pixel frames per second
    for VIDEO.  ``frame0`` (VIDEO) is the absolute latent-frame index of the
    first frame, or -1 to continue the running frame count of the DM region;
    ``step0`` (AUDIO / ACTION) is the index of the first token on its ladder.
    """
    region: int
    kind: int
    n_tokens: int = 0
    n_frames: int = 0
    n_views: int = 1
    grid_h: int = 0
    grid_w: int = 0
    rate: float = 0.0
    frame0: int = -1
    step0: int = 0

    def count(self) -> int:
        if self.kind == VIDEO:
            return self.n_frames * self.n_views * self.grid_h * self.grid_w
        return self.n_tokens


def text(n: int) -> Segment:
    return Segment(AR, TEXT, n_tokens=n)


def eos_bog() -> List[Segment]:
    return [Segment(AR, SPECIAL, n_tokens=1), Segment(AR, SPECIAL, n_tokens=1)]


def video(region: int, frames: int, views: int, gh: int, gw: int,
          fps: float = 24.0, frame0: int = -1) -> Segment:
    return Segment(region, VIDEO, n_frames=frames, n_views=views, grid_h=gh,
                   grid_w=gw, rate=fps, frame0=frame0)


def action(region: int, n: int, hz: float = 15.0, step0: int = 0) -> Segment:
    return Segment(region, ACTION, n_tokens=n, rate=hz, step0=step0)


def audio(region: int, n: int, tps: float = 25.0, step0: int = 0) -> Segment:
    return Segment(region, AUDIO, n_tokens=n, rate=tps, step0=step0)


def proprio(region: int, n: int = 1) -> Segment:
    return Segment(region, PROPRIO, n_tokens=n)


@dataclass(frozen=True)
class Workload:
    wid: int                       # workload id (seed root)
    name: str
    dtype: str                     # "fp32" or "bf16"
    n_heads: int
    head_dim: int
    hidden: int
    sections: Tuple[int, int, int]  # rotary pairs on the t / h / w axes
    segments: Tuple[Segment, ...]
    mask: int = AR_CAUSAL_DM_FULL
    sigmas: Tuple[float, ...] = ()
    theta: float = 10000.0
    n_kv_heads: int = 0            # key/value heads (0: n_heads)
    ffn: int = 0                   # MLP width of the whole layer (0: the attention path only)
    guidance: float = 0.0          # CFG weight of the guided step (0: unguided workload)
    # streaming (CHUNK_CAUSAL_KV) extras
    stream_views: int = 0
    stream_gh: int = 0
    stream_gw: int = 0
    stream_history_frames: int = 0
    stream_chunks: int = 0
    stream_steps: int = 0
    stream_text: int = 0
    notes: str = ""

    @property
    def n_tokens(self) -> int:
        return sum(s.count() for s in self.segments)

    @property
    def kv_heads(self) -> int:
        return self.n_kv_heads or self.n_heads


def _linear(n_steps: int) -> Tuple[float, ...]:
    return tuple(1.0 - k / n_steps for k in range(n_steps + 1))


def _build() -> List[Workload]:
    w = []
    # 1. Tiny, fp32: 32 text + EOS + BOG, 1 clean frame 4x6, 2 noisy frames
    #    4x6 and 8 action tokens = 114 tokens; one Euler step 1.0 -> 0.75.
    w.append(Workload(
        wid=0, name="tiny_fp32", dtype="fp32", n_heads=4, head_dim=64,
        hidden=256, sections=(8, 12, 12),
        segments=(text(32), *eos_bog(),
                  video(DM_CLEAN, 1, 1, 4, 6),
                  video(DM_NOISY, 2, 1, 4, 6), action(DM_NOISY, 8)),
        sigmas=(1.0, 0.75)))
    # 2. Policy-shaped, bf16: 256 text + EOS + BOG; clean 3 views x 1 frame
    #    12x20 + 1 proprio; noisy 3 views x 2 frames + 32 actions (vision
    #    before action inside a group); 10 linear Euler steps 1 -> 0.
    w.append(Workload(
        wid=1, name="policy_bf16", dtype="bf16", n_heads=24, head_dim=128,
        hidden=3072, sections=(16, 24, 24),
        segments=(text(256), *eos_bog(),
                  video(DM_CLEAN, 1, 3, 12, 20), proprio(DM_CLEAN, 1),
                  video(DM_NOISY, 2, 3, 12, 20), action(DM_NOISY, 32)),
        sigmas=_linear(10)))
    # 3. Text-to-video 480p-shaped: 512 text + EOS + BOG; 16 noisy latent
    #    frames on a 30x52 grid (24,960 tokens); no clean block.  The
    #    benchmark times one step, the first of a 40-step linear schedule.
    w.append(Workload(
        wid=2, name="t2v480p_bf16", dtype="bf16", n_heads=24, head_dim=128,
        hidden=3072, sections=(16, 24, 24),
        segments=(text(512), *eos_bog(), video(DM_NOISY, 16, 1, 30, 52)),
        sigmas=(1.0, 0.975)))
    # 4. Streaming chunk attention (Sim-Auto-shaped): 6 views at 12x20 per
    #    latent frame; cache = 256 text + EOS + BOG and 8 history frames;
    #    each query chunk is one latent frame; 4 steps per chunk, 16 chunks.
    w.append(Workload(
        wid=3, name="stream_chunk_bf16", dtype="bf16", n_heads=24,
        head_dim=128, hidden=3072, sections=(16, 24, 24),
        segments=(text(256), *eos_bog(),
                  video(DM_CLEAN, 8, 6, 12, 20, frame0=0),
                  video(DM_NOISY, 1, 6, 12, 20, frame0=8)),
        mask=CHUNK_CAUSAL_KV, sigmas=(1.0, 0.75, 0.5, 0.25, 0.0),
        stream_views=6, stream_gh=12, stream_gw=20, stream_history_frames=8,
        stream_chunks=16, stream_steps=4, stream_text=256))
    # 5. Long text-to-video 480p-shaped: 512 text + EOS + BOG; 1 clean
    #    conditioning frame and 48 noisy frames on 30x52 (76,954 tokens).
    w.append(Workload(
        wid=4, name="t2v480p_long_bf16", dtype="bf16", n_heads=24,
        head_dim=128, hidden=3072, sections=(16, 24, 24),
        segments=(text(512), *eos_bog(), video(DM_CLEAN, 1, 1, 30, 52),
                  video(DM_NOISY, 48, 1, 30, 52)),
        sigmas=(1.0, 0.975)))
    # 6. Grouped heads at the model table's Nano shape (32 query / 8 key-value
    #    heads of 128, hidden 4096) on the 480p text-to-video layout, with the
    #    guidance weight of the page's text-to-video settings (6).
    w.append(Workload(
        wid=5, name="nano_t2v480p_bf16", dtype="bf16", n_heads=32, head_dim=128,
        hidden=4096, sections=(16, 24, 24), n_kv_heads=8, guidance=6.0, ffn=12288,
        segments=(text(512), *eos_bog(), video(DM_NOISY, 16, 1, 30, 52)),
        sigmas=(1.0, 0.975)))
    # 7. Grouped heads at the model table's Super shape (64 query / 8
    #    key-value heads, hidden 5120, so heads of 5120 / 64 = 80 dims; FFN
    #    25600) on the same 480p text-to-video layout.  The 40 rotary pairs
    #    split t / h / w as 10 / 15 / 15, the D = 128 split scaled.
    w.append(Workload(
        wid=6, name="super_t2v480p_bf16", dtype="bf16", n_heads=64, head_dim=80,
        hidden=5120, sections=(10, 15, 15), n_kv_heads=8, guidance=6.0, ffn=25600,
        segments=(text(512), *eos_bog(), video(DM_NOISY, 16, 1, 30, 52)),
        sigmas=(1.0, 0.975)))
    return w


WORKLOADS: List[Workload] = _build()
BY_NAME = {wl.name: wl for wl in WORKLOADS}


def region_counts(segments) -> Tuple[int, int, int]:
    """(n_ar, n_clean, n_noisy): plain token counts per region tag."""
    c = [0, 0, 0]
    for s in segments:
        c[s.region] += s.count()
    return c[0], c[1], c[2]


# ----------------------------------------------------------------------------
# Seeded generators
# ----------------------------------------------------------------------------
# tensor ids
T_X, T_WQKV_AR, T_WQKV_DM, T_WO_AR, T_WO_DM, T_Q, T_K, T_V, T_LATENT = range(9)
T_X_BASE = 9  # the baseline (negative) prompt's AR rows of a guided step
# the whole layer: LayerNorm gamma / beta of each room (ln1, ln2), MLP matrices
T_LN1_G_AR, T_LN1_B_AR, T_LN1_G_DM, T_LN1_B_DM = 10, 11, 12, 13
T_LN2_G_AR, T_LN2_B_AR, T_LN2_G_DM, T_LN2_B_DM = 14, 15, 16, 17
T_UP_AR, T_UP_DM, T_DOWN_AR, T_DOWN_DM = 18, 19, 20, 21


def _rng(wid: int, tid: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([wid, tid, *extra])


def normal_f32(wid: int, tid: int, shape, std: float = 1.0, *extra: int) -> np.ndarray:
    x = _rng(wid, tid, *extra).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Tensor:
    """A seeded tensor: ``bits`` holds the exact stored bytes (uint16 for
    bf16, float32 for fp32); ``f32`` is the same values as float32."""
    dtype: str
    bits: np.ndarray
    f32: np.ndarray = field(repr=False)


def make(wid: int, tid: int, shape, dtype: str, std: float = 1.0, *extra: int) -> Tensor:
    x = normal_f32(wid, tid, shape, std, *extra)
    if dtype == "bf16":
        b = bf16_bits(x)
        return Tensor("bf16", b, bf16_to_f32(b))
    return Tensor("fp32", x, x)


def block_params(wl: Workload, dtype: Optional[str] = None) -> dict:
    """Seeded parameters of the whole layer for workload wl: LayerNorm gamma
    ~ 1 + N(0, 0.1^2) and beta ~ N(0, 0.1^2) (fp32), projection and MLP
    matrices ~ N(0, 0.02^2) in the workload's dtype.  Keys as oracle.block
    takes them; the (gamma, beta) pairs and matrices are Tensors."""
    dt = dtype or wl.dtype
    h, d, hid, hk, ffn = wl.n_heads, wl.head_dim, wl.hidden, wl.kv_heads, wl.ffn
    width = (h + 2 * hk) * d

    def ln(tg, tb):
        g = make(wl.wid, tg, (hid,), "fp32", 0.1)
        g = Tensor("fp32", g.f32 + np.float32(1.0), g.f32 + np.float32(1.0))
        return g, make(wl.wid, tb, (hid,), "fp32", 0.1)

    return {
        "ln1_ar": ln(T_LN1_G_AR, T_LN1_B_AR), "ln1_dm": ln(T_LN1_G_DM, T_LN1_B_DM),
        "ln2_ar": ln(T_LN2_G_AR, T_LN2_B_AR), "ln2_dm": ln(T_LN2_G_DM, T_LN2_B_DM),
        "qkv_ar": make(wl.wid, T_WQKV_AR, (hid, width), dt, 0.02),
        "qkv_dm": make(wl.wid, T_WQKV_DM, (hid, width), dt, 0.02),
        "o_ar": make(wl.wid, T_WO_AR, (h * d, hid), dt, 0.02),
        "o_dm": make(wl.wid, T_WO_DM, (h * d, hid), dt, 0.02),
        "up_ar": make(wl.wid, T_UP_AR, (hid, ffn), dt, 0.02),
        "up_dm": make(wl.wid, T_UP_DM, (hid, ffn), dt, 0.02),
        "down_ar": make(wl.wid, T_DOWN_AR, (ffn, hid), dt, 0.02),
        "down_dm": make(wl.wid, T_DOWN_DM, (ffn, hid), dt, 0.02),
    }


def to_torch(t: Tensor, device=None):
    """Move a seeded tensor's exact bytes into a torch tensor (no rounding)."""
    import torch
    if t.dtype == "bf16":
        out = torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16)
    else:
        out = torch.from_numpy(t.bits)
    return out.to(device) if device is not None else out


def to_numpy_f32(tt) -> np.ndarray:
    """Exact float32 values of a torch bf16/fp32 tensor (on any device)."""
    import torch
    tt = tt.detach().to("cpu").contiguous()
    if tt.dtype == torch.bfloat16:
        return bf16_to_f32(tt.view(torch.int16).numpy().view(np.uint16))
    return tt.to(torch.float32).numpy()
