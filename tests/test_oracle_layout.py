"""Pins of the oracle's packed-sequence layout (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def test_page_worked_time_steps():
    g = _golden("page_worked_values.json")["section_5_time_steps"]
    assert layout.video_tps(g["video_fps"]) == g["video_latent_tps"]
    assert layout.time_step(layout.video_tps(g["video_fps"])) == g["video_step"]
    assert layout.time_step(g["audio_tps"]) == g["audio_step"]
    assert layout.time_step(g["action_hz"]) == g["action_step"]


def test_page_worked_latent_shape():
    g = _golden("page_worked_values.json")["section_4_1_latent_shape"]
    assert layout.latent_frames(g["pixel_frames"]) == g["latent_frames"]
    gw, gh = layout.latent_grid(g["pixel_width"], g["pixel_height"])
    assert (gw, gh) == (g["latent_grid_w"], g["latent_grid_h"])
    segs = [W.text(4), *W.eos_bog(),
            W.video(W.DM_NOISY, g["latent_frames"], 1, gh, gw)]
    pos, reg, n_ar = layout.build(segs)
    assert int((reg == W.DM_NOISY).sum()) == g["visual_positions"]


@pytest.mark.parametrize("wl", W.WORKLOADS, ids=lambda w: w.name)
def test_workload_token_counts(wl):
    g = _golden("workload_token_counts.json")[wl.name]
    pos, reg, n_ar = layout.build(wl.segments)
    assert n_ar == g["n_ar"]
    assert int((reg == W.DM_CLEAN).sum()) == g["n_clean"]
    assert int((reg == W.DM_NOISY).sum()) == g["n_noisy"]
    assert len(reg) == pos.shape[0] == g["n"]
    assert pos.dtype == np.float32 and reg.dtype == np.uint8


def test_text_positions_are_1d_and_eos_bog_continue():
    wl = W.BY_NAME["tiny_fp32"]
    pos, reg, n_ar = layout.build(wl.segments)
    idx = np.arange(n_ar, dtype=np.float32)
    for a in range(3):
        np.testing.assert_array_equal(pos[:n_ar, a], idx)
    assert pos[32, 0] == 32 and pos[33, 0] == 33     # EOS, BOG
    assert (reg[:n_ar] == W.AR).all()


def test_dm_time_origin_gap():
    gap = _golden("page_worked_values.json")["section_5_ar_dm_time_gap"]
    for wl in W.WORKLOADS:
        pos, reg, n_ar = layout.build(wl.segments)
        dm_t = pos[n_ar:, 0]
        # the earliest DM time is the origin: next AR position + the gap
        assert float(dm_t.min()) == float(n_ar + gap)


def test_exact_rational_positions_for_action_and_audio():
    # t = t0 + 6k/TPS evaluated in exact rational arithmetic, rounded to
    # double then float32 (the canonical rounding), must equal the oracle.
    segs = [W.text(7), *W.eos_bog(), W.video(W.DM_CLEAN, 1, 1, 2, 3),
            W.audio(W.DM_NOISY, 50), W.action(W.DM_NOISY, 40)]
    pos, reg, n_ar = layout.build(segs)
    t0 = n_ar + 15000
    base = n_ar + 6
    for k in range(50):
        exact = Fraction(t0) + Fraction(6 * k, 25)
        assert pos[base + k, 0] == np.float32(float(exact))
        assert pos[base + k, 1] == 0 and pos[base + k, 2] == 0
    for k in range(40):
        exact = Fraction(t0) + Fraction(6 * k, 15)
        assert pos[base + 50 + k, 0] == np.float32(float(exact))
        assert pos[base + 50 + k, 1] == 0 and pos[base + 50 + k, 2] == 0


def test_video_grid_views_and_frame_continuity():
    wl = W.BY_NAME["policy_bf16"]
    pos, reg, n_ar = layout.build(wl.segments)
    t0 = n_ar + 15000
    clean = pos[reg == W.DM_CLEAN]
    noisy = pos[reg == W.DM_NOISY]
    vid_c = clean[:720]
    assert (vid_c[:, 0] == t0).all()
    # frame -> view -> row -> col; views tiled along w
    g = vid_c.reshape(3, 12, 20, 3)
    for v in range(3):
        np.testing.assert_array_equal(g[v, :, :, 1], np.repeat(np.arange(12), 20).reshape(12, 20))
        np.testing.assert_array_equal(g[v, :, :, 2], np.tile(np.arange(20) + 20 * v, (12, 1)))
    # proprio at the origin
    np.testing.assert_array_equal(clean[720], [t0, 0, 0])
    # noisy frames continue the frame count: 1, 2
    vid_n = noisy[:1440].reshape(2, 720, 3)
    assert (vid_n[0, :, 0] == t0 + 1).all() and (vid_n[1, :, 0] == t0 + 2).all()
    # 32 action tokens after the video of the noisy group
    act = noisy[1440:]
    assert act.shape[0] == 32 and (act[:, 1:] == 0).all()


def test_stream_layout_absolute_frames():
    wl = W.BY_NAME["stream_chunk_bf16"]
    pos, reg, n_ar = layout.build(wl.segments)
    t0 = n_ar + 15000
    hist = pos[reg == W.DM_CLEAN].reshape(8, 1440, 3)
    for f in range(8):
        assert (hist[f, :, 0] == t0 + f).all()
    chunk = pos[reg == W.DM_NOISY]
    assert (chunk[:, 0] == t0 + 8).all()
    assert chunk[:, 2].max() == 6 * 20 - 1


@pytest.mark.parametrize("segs", [
    [W.text(3), W.video(W.DM_NOISY, 1, 1, 2, 2), W.video(W.DM_CLEAN, 1, 1, 2, 2)],
    [W.text(3), W.action(W.DM_NOISY, 2), W.video(W.DM_NOISY, 1, 1, 2, 2)],
    [W.text(3), W.video(W.DM_NOISY, 1, 1, 2, 2), W.text(2)],
])
def test_order_violations_raise(segs):
    with pytest.raises(ValueError):
        layout.build(segs)
