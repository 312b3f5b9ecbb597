"""Pins of the oracle's whole MoT layer, oracle.block (CPU only).

* LayerNorm: explicit loops on a tiny input; with gamma = 1, beta = 0 every
  row has mean 0 and variance var / (var + eps); invariant to a per-row
  shift and positive scale of the input (up to eps); a constant row maps to
  beta.  Region split: the Generator's (gamma, beta) never touch AR rows.
* GELU: x Phi(x) against printed standard-normal CDF values (Phi(1), Phi(2),
  Phi(3), Phi(-1)); GELU(x) - GELU(-x) = x; GELU(0) = 0; GELU(x) -> x and
  -> 0 far from 0.
* MLP: explicit loops on a tiny input; the Generator's matrices never touch
  AR rows.
* Layer: with zero MLP matrices H2 = H1; with zero output-projection
  matrices H1 = X; H1 is the input plus oracle.denoiser's path applied to
  LN1(X); AR rows ignore every DM row; a uniform position shift changes
  nothing.  Each of these catches a mistake planted in a copy of the layer.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import block, denoiser

rng = np.random.default_rng(51)


def _r(*s):
    return rng.standard_normal(s)


# ---------------------------------------------------------------------------
def test_layer_norm_explicit_loops():
    x, g, b = _r(5, 7), _r(7), _r(7)
    got = block.layer_norm(x, g, b, eps=1e-3)
    for i in range(5):
        mu = sum(x[i]) / 7
        var = sum((t - mu) ** 2 for t in x[i]) / 7
        for j in range(7):
            assert abs(got[i, j] - ((x[i, j] - mu) / math.sqrt(var + 1e-3) * g[j] + b[j])) < 1e-13


def test_layer_norm_moments_and_invariances():
    x = _r(6, 64) * 3 + 1
    one, zero = np.ones(64), np.zeros(64)
    y = block.layer_norm(x, one, zero)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose(y.var(axis=1), var / (var + block.EPS), rtol=1e-12)
    g, b = _r(64), _r(64)
    a = block.layer_norm(x, g, b, eps=0.0)
    np.testing.assert_allclose(block.layer_norm(x * 2.5 + 7.0, g, b, eps=0.0), a, atol=1e-12)
    np.testing.assert_allclose(block.layer_norm(np.full((2, 64), 3.0), g, b), np.stack([b, b]), atol=1e-12)


def test_region_layer_norm_rooms():
    x = _r(9, 16)
    ar, dm = (_r(16), _r(16)), (_r(16), _r(16))
    y1 = block.region_layer_norm(x, ar, dm, 4)
    y2 = block.region_layer_norm(x, ar, (dm[0] * 3, dm[1] - 1), 4)
    np.testing.assert_array_equal(y1[:4], y2[:4])
    assert not np.allclose(y1[4:], y2[4:])
    np.testing.assert_allclose(y1[:4], block.layer_norm(x[:4], *ar), atol=1e-14)


def test_gelu_printed_normal_cdf_values():
    # standard normal CDF values as printed in statistical tables
    phi = {1.0: 0.8413447460685429, 2.0: 0.9772498680518208, 3.0: 0.9986501019683699,
           -1.0: 0.15865525393145707, 0.5: 0.6914624612740131}
    for x, p in phi.items():
        assert abs(block.gelu(np.array([x]))[0] - x * p) < 1e-15


def test_gelu_identities():
    x = _r(200) * 3
    np.testing.assert_allclose(block.gelu(x) - block.gelu(-x), x, atol=1e-14)
    assert block.gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(block.gelu(np.array([12.0, -12.0])), [12.0, 0.0], atol=1e-30)


def test_mlp_explicit_loops_and_rooms():
    u = _r(4, 3)
    ua, ud, da, dd = _r(3, 5), _r(3, 5), _r(5, 3), _r(5, 3)
    got = block.mlp(u, ua, ud, da, dd, 2)
    for i in range(4):
        w1, w2 = (ua, da) if i < 2 else (ud, dd)
        hid = [0.5 * s * (1 + math.erf(s / math.sqrt(2))) for s in
               (sum(u[i, e] * w1[e, c] for e in range(3)) for c in range(5))]
        for j in range(3):
            assert abs(got[i, j] - sum(hid[c] * w2[c, j] for c in range(5))) < 1e-13
    got2 = block.mlp(u, ua, ud * 2, da, dd + 1, 2)
    np.testing.assert_array_equal(got[:2], got2[:2])


# ---------------------------------------------------------------------------
H, D, HID, FFN, SECS, THETA = 2, 8, 16, 24, (1, 1, 2), 10000.0
N_AR, N_DM = 5, 7
N = N_AR + N_DM


def _params(seed, zero=()):
    r = np.random.default_rng(seed)
    p = {}
    for room in ("ar", "dm"):
        p["ln1_" + room] = (1 + 0.1 * r.standard_normal(HID), 0.1 * r.standard_normal(HID))
        p["ln2_" + room] = (1 + 0.1 * r.standard_normal(HID), 0.1 * r.standard_normal(HID))
        p["qkv_" + room] = r.standard_normal((HID, 3 * H * D)) * 0.3
        p["o_" + room] = r.standard_normal((H * D, HID)) * 0.3
        p["up_" + room] = r.standard_normal((HID, FFN)) * 0.3
        p["down_" + room] = r.standard_normal((FFN, HID)) * 0.3
    for k in zero:
        p[k] = np.zeros_like(p[k])
    return p


def _pos():
    ar = np.arange(N_AR, dtype=np.float32)
    dm = [(N_AR + 15000.0 + f, r_, c) for f in range(2) for r_ in range(2) for c in range(2)][:N_DM]
    return np.concatenate([np.stack([ar, ar, ar], 1), np.array(dm, np.float32)])


def _layer(layer_fn, X, p, pos=None):
    return layer_fn(X, p, _pos() if pos is None else pos, N_AR, H, D, SECS, THETA)


def _mutant(kind):
    def layer(X, p, pos, n_ar, nh, hd, secs, theta):
        q = dict(p)
        if kind == "ln_rooms_swapped":
            q["ln1_ar"], q["ln1_dm"] = p["ln1_dm"], p["ln1_ar"]
        if kind == "no_attention_residual":
            out = block.layer(X, q, pos, n_ar, nh, hd, secs, theta)
            return dict(out, h2=out["h2"] - X)
        if kind == "mlp_rooms_swapped":
            q["up_ar"], q["up_dm"] = p["up_dm"], p["up_ar"]
        if kind == "no_mlp_residual":
            out = block.layer(X, q, pos, n_ar, nh, hd, secs, theta)
            return dict(out, h2=out["h2"] - out["h1"])
        if kind == "post_norm":
            h1 = block.layer(X, dict(q, up_ar=0 * q["up_ar"], up_dm=0 * q["up_dm"]), pos, n_ar, nh, hd,
                             secs, theta)["h1"]
            h1n = block.region_layer_norm(h1, q["ln1_ar"], q["ln1_dm"], n_ar)
            return dict(h1=h1n, h2=h1n + block.mlp(h1n, q["up_ar"], q["up_dm"], q["down_ar"], q["down_dm"],
                                                   n_ar))
        if kind == "relu":
            out = block.layer(X, q, pos, n_ar, nh, hd, secs, theta)
            u2 = out["u2"]
            a = np.maximum(0, np.concatenate([u2[:n_ar] @ q["up_ar"], u2[n_ar:] @ q["up_dm"]]))
            return dict(out, h2=out["h1"] + np.concatenate([a[:n_ar] @ q["down_ar"], a[n_ar:] @ q["down_dm"]]))
        return block.layer(X, q, pos, n_ar, nh, hd, secs, theta)
    return layer


def pin_zero_mlp(layer_fn):
    X = np.random.default_rng(1).standard_normal((N, HID))
    out = _layer(layer_fn, X, _params(2, zero=("down_ar", "down_dm")))
    return np.abs(out["h2"] - out["h1"]).max() < 1e-13


def pin_zero_o(layer_fn):
    X = np.random.default_rng(3).standard_normal((N, HID))
    p = _params(4, zero=("o_ar", "o_dm"))
    out = _layer(layer_fn, X, p)
    ok = np.abs(out["h1"] - X).max() < 1e-13
    want = X + block.mlp(block.region_layer_norm(X, p["ln2_ar"], p["ln2_dm"], N_AR), p["up_ar"], p["up_dm"],
                         p["down_ar"], p["down_dm"], N_AR)
    return ok and np.abs(out["h2"] - want).max() < 1e-12


def pin_attention_path(layer_fn):
    X = np.random.default_rng(5).standard_normal((N, HID))
    p = _params(6)
    out = _layer(layer_fn, X, p)
    u1 = block.region_layer_norm(X, p["ln1_ar"], p["ln1_dm"], N_AR)
    z = denoiser.layer(u1, p["qkv_ar"], p["qkv_dm"], p["o_ar"], p["o_dm"], _pos(), N_AR, H, D, SECS,
                       THETA)["z"]
    return np.abs(out["h1"] - (X + z)).max() < 1e-12


def pin_ar_ignores_dm(layer_fn):
    X = np.random.default_rng(7).standard_normal((N, HID))
    X2 = X.copy()
    X2[N_AR:] = X2[N_AR:] * 3 - 1
    p = _params(8)
    return np.array_equal(_layer(layer_fn, X, p)["h2"][:N_AR], _layer(layer_fn, X2, p)["h2"][:N_AR])


def pin_shift(layer_fn):
    X = np.random.default_rng(9).standard_normal((N, HID))
    p = _params(10)
    a = _layer(layer_fn, X, p)["h2"]
    b = _layer(layer_fn, X, p, _pos() + np.array([11.0, 3.0, 2.0], np.float32))["h2"]
    return np.abs(a - b).max() < 1e-9


PINS = [pin_zero_mlp, pin_zero_o, pin_attention_path, pin_ar_ignores_dm, pin_shift]
MUTANTS = ["ln_rooms_swapped", "no_attention_residual", "mlp_rooms_swapped", "no_mlp_residual",
           "post_norm", "relu"]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_block_layer_satisfies_pin(pin):
    assert pin(block.layer)


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_block_mistake_fails_a_pin(kind):
    assert [p.__name__ for p in PINS if not p(_mutant(kind))], kind


def test_bf16_store_rounds_the_stored_tensors():
    X = np.random.default_rng(11).standard_normal((N, HID))
    p = _params(12)
    a = block.layer(X, p, _pos(), N_AR, H, D, SECS, THETA, store="bf16")
    for k in ("u1", "y", "q", "k", "o", "h1", "u2", "h2"):
        np.testing.assert_array_equal(denoiser.round_bf16(a[k]), a[k], err_msg=k)
    b = block.layer(X, p, _pos(), N_AR, H, D, SECS, THETA)
    assert 1e-4 < np.linalg.norm(a["h2"] - b["h2"]) / np.linalg.norm(b["h2"]) < 2e-2
