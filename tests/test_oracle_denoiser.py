"""Pins of the oracle's one-layer chain, oracle.denoiser (CPU only).

The chain composes pinned parts (projection, mRoPE, attention, Euler).  Its
composition is pinned here against sources other than itself:

* an independent build from explicit loops: projection as sums, mRoPE as a
  complex rotation, attention by the brute-force loops;
* the closed form with zero Q and K weights: scores vanish, every row
  averages the values it may read, so every DM velocity row equals
  mean(V) @ W_o_dm and AR row i equals mean(V[0..i]) @ W_o_ar;
* a uniform shift of every position leaves the layer unchanged (Q and K
  rotate together; "Cosmos 3 方法原理全解" §5);
* permuting the DM-noisy rows (with their positions) permutes the velocity
  rows the same way (DM rows read all keys, §3 O_DM).

Each pin is run against mistakes planted in a copy of the composition (K not
rotated, [Q|K|V] split order, rooms of either projection, the mask, V
rotated, the softmax scale, the mRoPE section order); every mistake fails at
least one pin.  The bf16-storage mode is pinned by exact rounding values and
by the storage points it rounds.
"""
import cmath
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention, denoiser, mrope, projection

H, D, HID = 2, 8, 16
SECS = (1, 1, 2)
THETA = 10000.0
N_AR, N_CLEAN, N_NOISY = 5, 3, 4
N = N_AR + N_CLEAN + N_NOISY


def _positions():
    ar = np.arange(N_AR, dtype=np.float32)
    pos = [np.stack([ar, ar, ar], 1)]
    t0 = N_AR + 15000.0
    dm = [(t0 + f, r, c) for f in range(2) for r in range(2) for c in range(2)][:N_CLEAN + N_NOISY]
    dm = [(t0 + 0.4 * k, 0, 0) for k in range(N_CLEAN + N_NOISY - len(dm))] + dm
    pos.append(np.array(dm, dtype=np.float32))
    return np.concatenate(pos)


def _inputs(seed=0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, HID))
    ws = [rng.standard_normal((HID, 3 * H * D)) * 0.3, rng.standard_normal((HID, 3 * H * D)) * 0.3,
          rng.standard_normal((H * D, HID)) * 0.3, rng.standard_normal((H * D, HID)) * 0.3]
    return X, ws, _positions()


def _z(layer_fn, X, ws, pos, n_ar=N_AR):
    return layer_fn(X, *ws, pos, n_ar, H, D, SECS, THETA)["z"]


# ---------------------------------------------------------------------------
# the independent build
def _loops_layer(X, w_qkv_ar, w_qkv_dm, w_o_ar, w_o_dm, pos, n_ar):
    n, hid = X.shape
    hd = H * D

    def proj(A, wa, wd):
        out = np.zeros((A.shape[0], wa.shape[1]))
        for r in range(A.shape[0]):
            w = wa if r < n_ar else wd
            for c in range(w.shape[1]):
                acc = 0.0
                for e in range(A.shape[1]):
                    acc += A[r, e] * w[e, c]
                out[r, c] = acc
        return out

    Y = proj(X, w_qkv_ar, w_qkv_dm)
    part = lambda s: np.array([[[Y[r, s * hd + h * D + e] for e in range(D)] for h in range(H)]
                               for r in range(n)])
    q, k, v = part(0), part(1), part(2)

    def rot(x):
        out = np.empty_like(x)
        half = D // 2
        for r in range(n):
            for h in range(H):
                for kk in range(half):
                    axis = 0 if kk < SECS[0] else (1 if kk < SECS[0] + SECS[1] else 2)
                    a = float(pos[r, axis]) * THETA ** (-2.0 * kk / D)
                    z = complex(x[r, h, kk], x[r, h, kk + half]) * cmath.exp(1j * a)
                    out[r, h, kk], out[r, h, kk + half] = z.real, z.imag
        return out

    o, _ = attention.attention_bruteforce(rot(q), rot(k), v, 0, W.AR_CAUSAL_DM_FULL, n_ar=n_ar)
    return proj(o.reshape(n, hd), w_o_ar, w_o_dm)


# ---------------------------------------------------------------------------
# planted mistakes: copies of the composition with one thing wrong
def _mutant(kind):
    def layer(X, wqa, wqd, woa, wod, pos, n_ar, nh, hd, secs, theta):
        n = X.shape[0]
        if kind == "qkv_rooms_swapped":
            y = projection.project(X, wqd, wqa, n_ar)
        else:
            y = projection.project(X, wqa, wqd, n_ar)
        q, k, v = projection.split_qkv(y, nh, hd)
        if kind == "k_from_v_columns":
            k, v = v, k
        if kind == "q_k_swapped":
            q, k = k, q
        s = secs[::-1] if kind == "sections_reversed" else secs
        qr = mrope.apply(q, pos, s, theta)
        kr = k if kind == "k_unrotated" else mrope.apply(k, pos, s, theta)
        if kind == "v_rotated":
            v = mrope.apply(v, pos, s, theta)
        nar_mask = {"dm_causal": n, "ar_full": 0}.get(kind, n_ar)
        scale = 1.0 if kind == "no_scale" else None
        o, lse = attention.attention(qr, kr, v, 0, W.AR_CAUSAL_DM_FULL, n_ar=nar_mask, scale=scale)
        o2 = o.reshape(n, nh * hd)
        if kind == "o_rooms_swapped":
            z = projection.project(o2, wod, woa, n_ar)
        elif kind == "o_all_generator":
            z = projection.project(o2, woa, wod, 0)
        else:
            z = projection.project(o2, woa, wod, n_ar)
        return dict(z=z)
    return layer


MUTANTS = ["qkv_rooms_swapped", "k_from_v_columns", "q_k_swapped", "sections_reversed",
           "k_unrotated", "v_rotated", "dm_causal", "ar_full", "no_scale", "o_rooms_swapped",
           "o_all_generator"]


# ---------------------------------------------------------------------------
# the pins, each a predicate on a layer function
def pin_loops(layer_fn):
    X, ws, pos = _inputs(1)
    return np.abs(_z(layer_fn, X, ws, pos) - _loops_layer(X, *ws, pos, N_AR)).max() < 1e-11


def pin_zero_qk_closed_form(layer_fn):
    X, ws, pos = _inputs(2)
    hd = H * D
    for w in ws[:2]:
        w[:, :2 * hd] = 0.0  # Q and K columns of both rooms
    z = _z(layer_fn, X, ws, pos)
    V = np.concatenate([X[:N_AR] @ ws[0][:, 2 * hd:], X[N_AR:] @ ws[1][:, 2 * hd:]])
    want_dm = V.mean(axis=0) @ ws[3]
    want_ar = np.stack([V[:i + 1].mean(axis=0) @ ws[2] for i in range(N_AR)])
    return (np.abs(z[N_AR:] - want_dm[None, :]).max() < 1e-12 and
            np.abs(z[:N_AR] - want_ar).max() < 1e-12)


def pin_shift_invariance(layer_fn):
    X, ws, pos = _inputs(3)
    shifted = pos + np.array([37.0, 5.0, 11.0], np.float32)
    return np.abs(_z(layer_fn, X, ws, pos) - _z(layer_fn, X, ws, shifted)).max() < 1e-9


def pin_dm_permutation(layer_fn):
    X, ws, pos = _inputs(4)
    r0 = N_AR + N_CLEAN
    perm = np.arange(N)
    perm[r0:] = r0 + np.random.default_rng(5).permutation(N_NOISY)
    z = _z(layer_fn, X, ws, pos)
    zp = _z(layer_fn, X[perm], ws, pos[perm])
    return np.abs(zp - z[perm]).max() < 1e-12


PINS = [pin_loops, pin_zero_qk_closed_form, pin_shift_invariance, pin_dm_permutation]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_layer_satisfies_pin(pin):
    assert pin(denoiser.layer)


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_fails_a_pin(kind):
    failed = [p.__name__ for p in PINS if not p(_mutant(kind))]
    assert failed, "mistake %s passes every pin" % kind


def test_independent_pins_catch_the_room_and_split_mistakes():
    # beyond the explicit-loop build, the closed form alone sees every
    # mistake of rooms and column order
    for kind in ("qkv_rooms_swapped", "k_from_v_columns", "o_rooms_swapped", "o_all_generator",
                 "dm_causal", "ar_full"):
        assert not pin_zero_qk_closed_form(_mutant(kind)), kind
    # and the shift invariance sees a one-sided rotation
    for kind in ("k_unrotated", "v_rotated"):
        assert not pin_shift_invariance(_mutant(kind)), kind


def test_step_velocity_is_the_noisy_rows_and_euler_applies():
    X, ws, pos = _inputs(6)
    r0 = N_AR + N_CLEAN
    x = X[r0:].astype(np.float32)
    out = denoiser.step(x, X[:r0], *ws, pos, N_AR, H, D, SECS, THETA, 1.0, 0.75)
    z = _loops_layer(np.concatenate([X[:r0], x.astype(np.float64)]), *ws, pos, N_AR)
    np.testing.assert_allclose(out["vel"], z[r0:], atol=1e-11)
    np.testing.assert_allclose(out["x_next"], x - 0.25 * z[r0:], atol=1e-11)


# ---------------------------------------------------------------------------
# bf16 storage mode
def test_round_bf16_ties_to_even_and_spacing():
    u = 2.0 ** -8  # half the bf16 spacing at 1
    vals = {1.0 + u: 1.0, 1.0 + 3 * u: 1.0 + 4 * u, 1.0 + 0.9 * u: 1.0, 1.0 + 1.1 * u: 1.0 + 2 * u,
            -(1.0 + 3 * u): -(1.0 + 4 * u), 3.0 * 2 ** -130: 3.0 * 2 ** -130, 0.0: 0.0,
            1.0 / 3.0: 0.333984375, 255.5: 256.0, 257.0: 256.0, 259.0: 260.0}
    for x, want in vals.items():
        assert denoiser.round_bf16(np.array([x]))[0] == want, x


def test_round_bf16_equals_bit_rounding_of_float32_values():
    # every float32 value is exact in float64, so rounding it from float64
    # must equal the RNE of its float32 bits
    x = np.random.default_rng(7).standard_normal(20000).astype(np.float32) * 37
    want = W.bf16_to_f32(W.bf16_bits(x)).astype(np.float64)
    np.testing.assert_array_equal(denoiser.round_bf16(x.astype(np.float64)), want)


def test_bf16_store_rounds_exactly_the_storage_points():
    X, ws, pos = _inputs(8)
    a = denoiser.layer(X, *ws, pos, N_AR, H, D, SECS, THETA, store="bf16")
    b = denoiser.layer(X, *ws, pos, N_AR, H, D, SECS, THETA)
    for name in ("y", "q", "k", "v", "o", "z"):
        np.testing.assert_array_equal(denoiser.round_bf16(a[name]), a[name], err_msg=name)
        assert not np.array_equal(b[name], denoiser.round_bf16(b[name])), name
    # each stage of the stored chain is the unrounded stage applied to the
    # stored tensors before it, then rounded
    y = denoiser.round_bf16(projection.project(X, ws[0], ws[1], N_AR))
    np.testing.assert_array_equal(a["y"], y)
    q, k, v = projection.split_qkv(y, H, D)
    np.testing.assert_array_equal(a["k"], denoiser.round_bf16(mrope.apply(k, pos, SECS, THETA)))
    o, _ = attention.attention(a["q"], a["k"], v, 0, W.AR_CAUSAL_DM_FULL, n_ar=N_AR)
    np.testing.assert_array_equal(a["o"], denoiser.round_bf16(o))
    z = projection.project(a["o"].reshape(N, H * D), ws[2], ws[3], N_AR)
    np.testing.assert_array_equal(a["z"], denoiser.round_bf16(z))
    # the rounding stays within bf16's relative half-spacing per stored value,
    # so the stored chain is close to the unrounded one
    rel = np.linalg.norm(a["z"] - b["z"]) / np.linalg.norm(b["z"])
    assert 1e-4 < rel < 2e-2
