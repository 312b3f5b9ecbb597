"""Packed-sequence layout: region tags and (t, h, w) mRoPE coordinates.

Follows "Cosmos 3 方法原理全解":

* §2: the sequence is [AR text ..., EOS, BOG, DM-clean ..., DM-noisy ...];
  inside the DM region all clean conditions come first, then all noisy
  targets, and inside each group the order is vision, audio, action.
* §5: text tokens use t = h = w (ordinary 1D RoPE); video uses t for time and
  (h, w) for the latent grid; audio and action use t only with h = w = 0.
  Time steps scale with the real rate: TPS_video = FPS / 4 and Δt = 6 / TPS,
  so 24 FPS video steps by 1, 25 token/s audio by 0.24, 15 Hz action by 0.4.
  The DM time axis starts 15000 after the AR one (an offset, no tokens).
  Clean prefix and noisy future share one time axis.
* §4.1: latent video shape, T_latent = 1 + (F - 1) / 4, one latent position
  per 32x32 pixels.

Readings where the pages are silent (each listed in the design notes):

* EOS and BOG are AR tokens and continue the text positions.
* The DM time origin is t0 = n_ar + 15000 (the next AR position, advanced by
  the gap).
* A token k on a rate-r ladder sits at t0 + (6 k) / TPS, evaluated in double
  as ``t0 + (6.0*k)/tps`` and rounded once to float32.  Video frame f uses
  the same rule with TPS = FPS/4; proprioception sits at t0.
* Video grid coordinates are 0-based; several camera views are tiled along w
  (w = view * W + col) and ordered frame -> view -> row -> col.
* Latent frames are counted continuously through the DM video groups unless
  a group gives its absolute first frame (streaming).
"""
from __future__ import annotations

import numpy as np

from workloads import (AR, DM_CLEAN, DM_NOISY, TEXT, SPECIAL, VIDEO, AUDIO,
                       ACTION, PROPRIO)

AR_DM_TIME_GAP = 15000.0      # §5, first extra rule
VIDEO_TEMPORAL_STRIDE = 4     # §4.1 / §5: 4 pixel frames per latent frame
PIXELS_PER_LATENT = 32        # §4.1: one latent position per 32x32 pixels


def latent_frames(n_pixel_frames: int) -> int:
    """T_latent = 1 + (F - 1) / 4 (§4.1); the prime frame is coded alone."""
    if (n_pixel_frames - 1) % VIDEO_TEMPORAL_STRIDE:
        raise ValueError("frame count must be 1 + 4k")
    return 1 + (n_pixel_frames - 1) // VIDEO_TEMPORAL_STRIDE


def latent_grid(width_px: int, height_px: int, px: int = PIXELS_PER_LATENT):
    """(grid_w, grid_h) for a width x height video (§4.1)."""
    return width_px // px, height_px // px


def time_step(tps: float) -> float:
    """Δt = 6 / TPS (§5)."""
    return 6.0 / tps


def video_tps(fps: float) -> float:
    """TPS_video = FPS / 4 (§5)."""
    return fps / 4.0


def _dm_class(kind: int) -> int:
    # order inside a DM group: vision, audio, action (proprio is state and
    # sits with action)
    return {VIDEO: 0, AUDIO: 1, ACTION: 2, PROPRIO: 2}[kind]


def check_order(segments) -> None:
    """Raise ValueError unless the segment list follows the §2 order."""
    seen_dm = False
    last_region = AR
    last_class = -1
    for s in segments:
        if s.region == AR:
            if seen_dm:
                raise ValueError("AR segment after a DM segment")
            if s.kind not in (TEXT, SPECIAL):
                raise ValueError("AR region holds text / special tokens only")
            continue
        if s.region not in (DM_CLEAN, DM_NOISY):
            raise ValueError("unknown region")
        if s.kind not in (VIDEO, AUDIO, ACTION, PROPRIO):
            raise ValueError("DM region holds video / audio / action / proprio")
        seen_dm = True
        if s.region < last_region:
            raise ValueError("clean conditions must precede noisy targets")
        if s.region != last_region:
            last_class = -1
        c = _dm_class(s.kind)
        if c < last_class:
            raise ValueError("DM group order is vision, audio, action")
        last_region, last_class = s.region, c


def build(segments):
    """Return (pos[N,3] float32, region[N] uint8, n_ar).

    Positions are computed in float64 and rounded once to float32.
    """
    check_order(segments)
    pos = []
    reg = []
    n_ar = sum(s.count() for s in segments if s.region == AR)
    t0 = float(n_ar) + AR_DM_TIME_GAP
    i_ar = 0
    frames_seen = 0
    for s in segments:
        n = s.count()
        if n <= 0:
            raise ValueError("empty segment")
        if s.region == AR:
            for _ in range(n):
                p = float(i_ar)
                pos.append((p, p, p))
                reg.append(AR)
                i_ar += 1
            continue
        if s.kind == VIDEO:
            f0 = s.frame0 if s.frame0 >= 0 else frames_seen
            tps = video_tps(s.rate)
            for f in range(s.n_frames):
                t = t0 + (6.0 * (f0 + f)) / tps
                for v in range(s.n_views):
                    for r in range(s.grid_h):
                        for c in range(s.grid_w):
                            pos.append((t, float(r), float(v * s.grid_w + c)))
                            reg.append(s.region)
            frames_seen = f0 + s.n_frames
        elif s.kind in (AUDIO, ACTION):
            for k in range(n):
                t = t0 + (6.0 * (s.step0 + k)) / s.rate
                pos.append((t, 0.0, 0.0))
                reg.append(s.region)
        elif s.kind == PROPRIO:
            for _ in range(n):
                pos.append((t0, 0.0, 0.0))
                reg.append(s.region)
    p64 = np.array(pos, dtype=np.float64).reshape(-1, 3)
    return p64.astype(np.float32), np.array(reg, dtype=np.uint8), n_ar
