"""Helpers for the GPU parity tests (not a test module)."""
import sys

import numpy as np
import pytest

BF16_MAX_ABS = 2e-2   # bf16 in / fp32 accumulate vs the fp64 oracle
BF16_REL_L2 = 5e-3
F32_MAX_ABS = 1e-4    # fp32 paths (tiny workload): the same contract holds;
F32_REL_L2 = 1e-5     # these tighter bounds document the fp32 arithmetic


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


def to_np(t):
    from workloads import to_numpy_f32
    return to_numpy_f32(t)
