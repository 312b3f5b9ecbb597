"""Pins of the oracle's region-split projection, Euler step, streaming cache
and one-layer chain (CPU only)."""
import numpy as np
import pytest

import workloads as W
from oracle import attention, denoiser, euler, layout, mrope, projection, streaming


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_projection_equal_rooms_is_plain_matmul():
    x, w = _rand((13, 8), 1), _rand((8, 5), 2)
    np.testing.assert_allclose(projection.project(x, w, w, 6), np.matmul(x, w), atol=1e-13)


def test_projection_bruteforce():
    x, wa, wd = _rand((5, 4), 3), _rand((4, 3), 4), _rand((4, 3), 5)
    n_ar = 2
    y = projection.project(x, wa, wd, n_ar)
    for r in range(5):
        w = wa if r < n_ar else wd
        for c in range(3):
            acc = 0.0
            for e in range(4):
                acc += x[r, e] * w[e, c]
            assert abs(y[r, c] - acc) < 1e-13


def test_projection_ar_rows_ignore_generator_weights():
    x, wa, wd = _rand((9, 4), 6), _rand((4, 6), 7), _rand((4, 6), 8)
    y1 = projection.project(x, wa, wd, 4)
    y2 = projection.project(x, wa, wd * 3 + 1, 4)
    np.testing.assert_array_equal(y1[:4], y2[:4])
    assert not np.allclose(y1[4:], y2[4:])


def test_split_qkv_columns():
    y = np.arange(2 * 3 * 2 * 4).reshape(2, 24).astype(float)
    q, k, v = projection.split_qkv(y, 2, 4)
    np.testing.assert_array_equal(q[1, 1], y[1, 4:8])
    np.testing.assert_array_equal(k[0, 0], y[0, 8:12])
    np.testing.assert_array_equal(v[1, 0], y[1, 16:20])


def test_euler_zero_velocity_is_identity():
    x = _rand((100,), 9).astype(np.float32)
    np.testing.assert_array_equal(euler.step(x, np.zeros_like(x), 1.0, 0.75), x)


def test_euler_exact_on_rectified_flow_path():
    # x_sigma = sigma*eps + (1-sigma)*x0 with the true velocity v* = eps - x0:
    # any schedule from sigma = 1 (pure noise) to 0 lands exactly on x0.
    eps, x0 = _rand((64,), 10), _rand((64,), 11)
    for sched in (euler.linear_schedule(10), [1.0, 0.75, 0.5, 0.25, 0.0], [1.0, 0.0]):
        x = euler.flow_path(eps, x0, sched[0])
        for s, sn in zip(sched[:-1], sched[1:]):
            x = euler.step(x, euler.true_velocity(eps, x0), s, sn)
            np.testing.assert_allclose(x, euler.flow_path(eps, x0, np.float32(sn)), atol=1e-12)
        np.testing.assert_allclose(x, x0, atol=1e-12)


def test_euler_linear_in_velocity():
    x, v1, v2 = _rand((30,), 12), _rand((30,), 13), _rand((30,), 14)
    a = euler.step(x, v1 + v2, 0.6, 0.2)
    b = euler.step(x, v1, 0.6, 0.2) + euler.step(x, v2, 0.6, 0.2) - x
    np.testing.assert_allclose(a, b, atol=1e-13)


def test_stream_cache_equals_chronological_attention():
    # a ring-ordered cache gives the same outputs as the keys laid out in
    # time order (softmax attention is invariant to the order of its keys)
    rng = np.random.default_rng(15)
    h, d, ft, slots, npre = 2, 8, 6, 3, 4
    secs = (1, 1, 2)
    pk, pv = rng.standard_normal((npre, h, d)), rng.standard_normal((npre, h, d))
    ppos = np.stack([np.arange(npre)] * 3, 1).astype(np.float32)
    frames = {f: (rng.standard_normal((ft, h, d)), rng.standard_normal((ft, h, d)))
              for f in range(slots)}
    fpos = lambda f: np.stack([np.full(ft, 100 + f), np.arange(ft) // 3, np.arange(ft) % 3], 1).astype(np.float32)
    hk = np.concatenate([frames[f][0] for f in range(slots)])
    hv = np.concatenate([frames[f][1] for f in range(slots)])
    hpos = np.concatenate([fpos(f) for f in range(slots)])
    cache = streaming.RollingCache(pk, pv, ppos, hk, hv, hpos, ft, secs, 1e4)
    for c in range(5):
        f = slots + c
        q, k, v = (rng.standard_normal((ft, h, d)) for _ in range(3))
        o, kr = cache.attend(q, k, v, fpos(f))
        # chronological reference: prefix, the last `slots` frames, chunk
        hist = list(range(f - slots, f))
        kk = np.concatenate([pk] + [frames[g][0] for g in hist] + [k])
        vv = np.concatenate([pv] + [frames[g][1] for g in hist] + [v])
        pp = np.concatenate([ppos] + [fpos(g) for g in hist] + [fpos(f)])
        kk = mrope.apply(kk, pp, secs, 1e4)
        qq = mrope.apply(q, fpos(f), secs, 1e4)
        want, _ = attention.attention(qq, kk, vv, 0, W.AR_CAUSAL_DM_FULL, n_ar=0)
        np.testing.assert_allclose(o, want, atol=1e-12)
        frames[f] = (k, v)
        cache.append(c, kr, v)


def test_one_layer_chain_ar_rows_ignore_the_noisy_latent():
    wl = W.BY_NAME["tiny_fp32"]
    pos, reg, n_ar = layout.build(wl.segments)
    n = len(reg)
    n_noisy = int((reg == W.DM_NOISY).sum())
    hid, h, d = wl.hidden, wl.n_heads, wl.head_dim
    X = _rand((n, hid), 16)
    ws = [_rand((hid, 3 * h * d), s) * 0.02 for s in (17, 18)] + \
         [_rand((h * d, hid), s) * 0.02 for s in (19, 20)]
    x = X[n - n_noisy:].astype(np.float32)
    a = denoiser.step(x, X[:n - n_noisy], *ws, pos, n_ar, h, d, wl.sections, wl.theta, 1.0, 0.75)
    b = denoiser.step(x * 2 + 1, X[:n - n_noisy], *ws, pos, n_ar, h, d, wl.sections, wl.theta, 1.0, 0.75)
    np.testing.assert_array_equal(a["z"][:n_ar], b["z"][:n_ar])
    assert a["x_next"].shape == x.shape
    np.testing.assert_allclose(a["x_next"], x - 0.25 * a["vel"], atol=1e-12)
