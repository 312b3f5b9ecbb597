"""Pins of the oracle's classifier-free guidance (oracle.cfg) and of grouped
key/value heads in oracle.attention (CPU only).

CFG ("Cosmos 3 方法原理全解" §7.2 CFG equation, §7.3 generation loop):
* w = 1 gives v_cond and w = 0 gives v_base (exactly on dyadic values); the
  combination is
  the affine map (1 - w) v_base + w v_cond;
* with both branches' velocity equal to the rectified-flow velocity
  eps - x0 (§6.3), the guided Euler sampler lands on x0 for any w;
* one guided step of the one-layer chain: identical prompts give v_cond for
  any w, w = 1 equals the unguided chain with the condition prompt, w = 0
  the chain with the baseline prompt, and the guided x_next is linear in w.
Planted mistakes in copies of ``combine`` each fail one of these.

Grouped heads (§12.4 model table: Q / KV heads 16/8, 32/8, 64/8):
* GQA equals multi-head attention with each key/value head repeated for its
  group of query heads (the multi-head form is pinned by brute force);
* the explicit-loop evaluation agrees, in both mask modes;
* attention_rows with the grouped head map agrees.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention, cfg, denoiser, euler

rng = np.random.default_rng(41)


def _r(*shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------
# CFG
def test_combine_end_points():
    vc, vb = _r(50), _r(50)
    # w = 0 is exact; w = 1 rounds the difference and the sum once each
    np.testing.assert_array_equal(cfg.combine(vc, vb, 0.0), vb)
    np.testing.assert_allclose(cfg.combine(vc, vb, 1.0), vc, rtol=0, atol=1e-15 * np.abs(vb).max() * 4)
    # on dyadic values both are exact
    vc, vb = rng.integers(-64, 64, 40) / 8.0, rng.integers(-64, 64, 40) / 8.0
    np.testing.assert_array_equal(cfg.combine(vc, vb, 1.0), vc)


def test_combine_is_the_affine_map_in_w():
    # dyadic values: every product and sum below is exact in float64
    vc = rng.integers(-64, 64, 40) / 8.0
    vb = rng.integers(-64, 64, 40) / 8.0
    for w in (0.5, 2.0, 3.0, 6.0, -1.5, 1.5):
        np.testing.assert_array_equal(cfg.combine(vc, vb, w), (1 - w) * vb + w * vc)


def test_guided_sampler_exact_on_rectified_flow_path():
    eps, x0 = _r(64), _r(64)
    vstar = euler.true_velocity(eps, x0)
    for w in (1.0, 3.0, 6.0):
        for sched in (euler.linear_schedule(10), [1.0, 0.75, 0.5, 0.25, 0.0]):
            x = euler.flow_path(eps, x0, 1.0)
            for s, sn in zip(sched[:-1], sched[1:]):
                x = cfg.euler_step(x, vstar, vstar, w, s, sn)
            np.testing.assert_allclose(x, x0, atol=1e-12)


def _mutant(kind):
    def combine(vc, vb, w):
        vc, vb = np.asarray(vc, np.float64), np.asarray(vb, np.float64)
        if kind == "sign":
            return vb + w * (vb - vc)
        if kind == "w_on_base":
            return vc + w * (vc - vb)
        if kind == "no_base":
            return w * (vc - vb)
        if kind == "scaled":
            return w * vc + vb
    return combine


@pytest.mark.parametrize("kind", ["sign", "w_on_base", "no_base", "scaled"])
def test_planted_combine_mistakes_fail_the_end_points(kind):
    vc, vb = rng.integers(-64, 64, 20) / 8.0, rng.integers(-64, 64, 20) / 8.0
    f = _mutant(kind)
    ok = (np.array_equal(f(vc, vb, 1.0), vc) and np.array_equal(f(vc, vb, 0.0), vb))
    assert not ok


H, D, HID, SECS, THETA = 2, 8, 16, (1, 1, 2), 10000.0
N_AR, N_CLEAN, N_NOISY = 5, 3, 4


def _chain_inputs(seed, n_kv=None):
    r = np.random.default_rng(seed)
    hk = H if n_kv is None else n_kv
    qkv = (H + 2 * hk) * D
    ws = [r.standard_normal((HID, qkv)) * 0.3, r.standard_normal((HID, qkv)) * 0.3,
          r.standard_normal((H * D, HID)) * 0.3, r.standard_normal((H * D, HID)) * 0.3]
    pos = np.concatenate([np.repeat(np.arange(N_AR, dtype=np.float32)[:, None], 3, 1),
                          np.array([[N_AR + 15000.0 + f, r_, c] for f in range(2) for r_ in range(2)
                                    for c in range(2)][:N_CLEAN + N_NOISY], np.float32)])
    return (r.standard_normal((N_AR, HID)), r.standard_normal((N_AR, HID)),
            r.standard_normal((N_CLEAN, HID)), r.standard_normal((N_NOISY, HID)).astype(np.float32),
            ws, pos)


def _step(x, Xc, Xb, Xcl, ws, pos, w, n_kv=None):
    return cfg.step(x, Xc, Xb, Xcl, *ws, pos, N_AR, H, D, SECS, THETA, w, 1.0, 0.75, n_kv_heads=n_kv)


def test_cfg_step_identical_prompts_give_v_cond():
    Xc, _, Xcl, x, ws, pos = _chain_inputs(1)
    for w in (0.0, 3.0, 6.0):
        out = _step(x, Xc, Xc, Xcl, ws, pos, w)
        np.testing.assert_allclose(out["vel"], out["vel_cond"], atol=1e-12)


def test_cfg_step_end_points_are_the_unguided_chains():
    Xc, Xb, Xcl, x, ws, pos = _chain_inputs(2)
    for w, X_ar in ((1.0, Xc), (0.0, Xb)):
        out = _step(x, Xc, Xb, Xcl, ws, pos, w)
        ref = denoiser.step(x, np.concatenate([X_ar, Xcl]), *ws, pos, N_AR, H, D, SECS, THETA,
                            1.0, 0.75)
        np.testing.assert_allclose(out["vel"], ref["vel"], atol=1e-12)
        np.testing.assert_allclose(out["x_next"], ref["x_next"], atol=1e-12)
    # the two branches really differ
    out = _step(x, Xc, Xb, Xcl, ws, pos, 3.0)
    assert np.abs(out["vel_cond"] - out["vel_base"]).max() > 1e-3


def test_cfg_step_x_next_is_linear_in_w():
    Xc, Xb, Xcl, x, ws, pos = _chain_inputs(3)
    a, b, c = (_step(x, Xc, Xb, Xcl, ws, pos, w)["x_next"] for w in (1.0, 3.0, 5.0))
    np.testing.assert_allclose(b, (a + c) / 2, atol=1e-12)


def test_cfg_step_rejects_unequal_prompt_lengths():
    Xc, Xb, Xcl, x, ws, pos = _chain_inputs(4)
    with pytest.raises(ValueError):
        _step(x, Xc, Xb[:-1], Xcl, ws, pos, 2.0)


# ---------------------------------------------------------------------------
# grouped key/value heads
@pytest.mark.parametrize("h,hk", [(4, 2), (4, 1), (8, 4), (6, 3), (4, 4)])
@pytest.mark.parametrize("mode", [W.AR_CAUSAL_DM_FULL, W.CHUNK_CAUSAL_KV])
def test_gqa_equals_mha_with_repeated_kv_heads(h, hk, mode):
    nq, nk, d = 30, 44, 8
    q, k, v = _r(nq, h, d), _r(nk, hk, d), _r(nk, hk, d)
    kw = dict(n_ar=9) if mode == W.AR_CAUSAL_DM_FULL else dict(n_prefix=6, chunk_len=5)
    q0 = nk - nq
    got, lse = attention.attention(q, k, v, q0, mode, **kw)
    rep = h // hk
    want, lse2 = attention.attention(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), q0, mode, **kw)
    np.testing.assert_allclose(got, want, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)
    bf, _ = attention.attention_bruteforce(q, k, v, q0, mode, **kw)
    np.testing.assert_allclose(got, bf, atol=1e-12)


def test_gqa_head_map_and_rows():
    assert [attention.kv_head(h, 32, 8) for h in range(32)] == [h // 4 for h in range(32)]
    assert [attention.kv_head(h, 24, 24) for h in range(24)] == list(range(24))
    with pytest.raises(ValueError):
        attention.kv_head(0, 6, 4)
    q, k, v = _r(20, 8, 8), _r(20, 2, 8), _r(20, 2, 8)
    full, _ = attention.attention(q, k, v, 0, W.AR_CAUSAL_DM_FULL, n_ar=7)
    rows, heads = [0, 3, 7, 19], [1, 5, 6]
    got = attention.attention_rows(q[rows], k, v, rows, heads, 0, W.AR_CAUSAL_DM_FULL, n_ar=7,
                                   kv_heads=[attention.kv_head(hh, 8, 2) for hh in heads])
    np.testing.assert_allclose(got, full[rows][:, heads], atol=1e-13)


def test_gqa_chain_layer_and_cfg():
    # the one-layer chain with grouped heads: equal to the multi-head chain
    # whose K and V weight columns repeat each group's head
    hk = 1
    Xc, Xb, Xcl, x, ws, pos = _chain_inputs(5, n_kv=hk)
    X = np.concatenate([Xc, Xcl, x.astype(np.float64)])
    got = denoiser.layer(X, *ws, pos, N_AR, H, D, SECS, THETA, n_kv_heads=hk)["z"]

    def widen(wq):
        q, k, v = wq[:, :H * D], wq[:, H * D:(H + hk) * D], wq[:, (H + hk) * D:]
        rep = lambda t: np.repeat(t.reshape(HID, hk, D), H // hk, axis=1).reshape(HID, H * D)
        return np.concatenate([q, rep(k), rep(v)], axis=1)

    ws_mha = [widen(ws[0]), widen(ws[1]), ws[2], ws[3]]
    want = denoiser.layer(X, *ws_mha, pos, N_AR, H, D, SECS, THETA)["z"]
    np.testing.assert_allclose(got, want, atol=1e-12)
    out = _step(x, Xc, Xb, Xcl, ws, pos, 3.0, n_kv=hk)
    assert out["vel"].shape == x.shape
