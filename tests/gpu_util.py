"""Helpers for the GPU parity tests (not a test module)."""
import sys

import numpy as np
import pytest

BF16_MAX_ABS = 2e-2   # bf16 in / fp32 accumulate vs the fp64 oracle
BF16_REL_L2 = 5e-3
F32_MAX_ABS = 1e-4    # fp32 paths (tiny workload): the same contract holds;
F32_REL_L2 = 1e-5     # these tighter bounds document the fp32 arithmetic
# The bf16 attention kernel's LSE: its row sum adds the bf16-rounded P that
# the PV product uses, each within a relative 2^-8 (the unit roundoff of an
# 8-bit significand), so the sum and the LSE are off by at most
# ln(1 + 2^-8) = 3.9e-3, plus the fp32 error of the scores (~1e-4).
BF16_LSE_ATOL = 4e-3


def device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def errors(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    d = got - want
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    den = float(np.sqrt((want ** 2).sum()))
    rel = float(np.sqrt((d ** 2).sum()) / den) if den > 0 else float(np.sqrt((d ** 2).sum()))
    return max_abs, rel


def assert_parity(got, want, dtype="bf16", what=""):
    ma, rl = errors(got, want)
    if dtype == "bf16":
        lim_a, lim_r = BF16_MAX_ABS, BF16_REL_L2
    else:
        lim_a, lim_r = F32_MAX_ABS, F32_REL_L2
    say("  parity %-28s max_abs=%.3e rel_l2=%.3e (limits %.0e / %.0e)" % (what, ma, rl, lim_a, lim_r))
    assert ma <= lim_a and rl <= lim_r, (what, ma, rl)
    return ma, rl


def bf16_spacing(v):
    """One bfloat16 spacing at |v| (8 significant bits), elementwise."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 7), 0.0)


def assert_parity_stored(got, want, what="", spacings=1):
    """The bf16 contract for a tensor stored in bf16 whose values may be
    large: relative L2 <= 5e-3, and per element |got - want| <= max(2e-2,
    `spacings` bf16 spacings at the larger of |got| and |want|).  Storing a
    value in bf16 moves it by up to half a spacing, which passes 2e-2 once
    |value| >= 8, and two stored results may sit a spacing apart from
    |value| >= 4; where they straddle a power of two, that spacing is the
    upper binade's.  A stored value that adds to an earlier stored value
    compared end to end (H2 = round(H1 + delta) against the oracle's own H1)
    carries that one's spacing too: spacings=2."""
    ma, rl = errors(got, want)
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    d = np.abs(g - w)
    allow = np.maximum(BF16_MAX_ABS, spacings * bf16_spacing(np.maximum(np.abs(g), np.abs(w))))
    worst = float((d / allow).max()) if d.size else 0.0
    say("  parity %-28s max_abs=%.3e rel_l2=%.3e worst/allowance=%.2f (stored bf16)" % (what, ma, rl, worst))
    assert rl <= BF16_REL_L2 and worst <= 1.0, (what, ma, rl, worst)
    return ma, rl


def to_np(t):
    from workloads import to_numpy_f32
    return to_numpy_f32(t)


def stream_workload(size):
    """The streaming workload ("stream_chunk_bf16"), or ("mini") the same
    structure reduced to 8-token frames of 2 heads of 64 with an 8-token
    text prefix and 11 chunks, which still wrap the 8-slot ring."""
    import dataclasses

    import workloads as W
    full = W.BY_NAME["stream_chunk_bf16"]
    if size == "stream_chunk_bf16":
        return full
    assert size == "mini", size
    return dataclasses.replace(
        full, name="stream_mini_bf16", n_heads=2, head_dim=64, hidden=128, sections=(8, 12, 12),
        segments=(W.text(6), *W.eos_bog(), W.video(W.DM_CLEAN, 8, 1, 2, 4, frame0=0),
                  W.video(W.DM_NOISY, 1, 1, 2, 4, frame0=8)),
        stream_views=1, stream_gh=2, stream_gw=4, stream_chunks=11, stream_text=6)
