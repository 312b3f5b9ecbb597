"""Pins of the oracle's 3D mRoPE (CPU only)."""
import numpy as np
import pytest

from oracle import mrope

SECTIONS = {64: (8, 12, 12), 80: (10, 15, 15), 128: (16, 24, 24)}


def _rope1d_complex(x, p, theta):
    """Textbook 1D RoPE in complex form, written independently of the oracle:
    z_k = x_k + i x_{k+D/2};  z_k <- z_k * exp(i * p * theta^(-2k/D))."""
    n, h, d = x.shape
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    w = np.array([theta ** (-(2.0 * kk) / d) for kk in range(half)])
    rot = np.exp(1j * np.outer(p, w))[:, None, :]
    z = z * rot
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("d", [64, 80, 128])
def test_text_positions_reduce_to_1d_rope(d):
    rng = np.random.default_rng(1)
    n = 40
    x = rng.standard_normal((n, 3, d))
    p = np.arange(n, dtype=np.float32) * 7 + 3
    pos = np.stack([p, p, p], axis=1)
    got = mrope.apply(x, pos, SECTIONS[d], 10000.0)
    want = _rope1d_complex(x, p.astype(np.float64), 10000.0)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("d", [64, 80, 128])
def test_relative_shift_invariance_at_dm_positions(d):
    rng = np.random.default_rng(2)
    n = 24
    q = rng.standard_normal((n, 2, d))
    k = rng.standard_normal((n, 2, d))
    pos = np.stack([15514 + rng.integers(0, 48, n), rng.integers(0, 30, n),
                    rng.integers(0, 52, n)], axis=1).astype(np.float32)
    shift = np.array([37, 5, 11], dtype=np.float32)
    s0 = np.einsum("ihd,jhd->hij", mrope.apply(q, pos, SECTIONS[d], 1e4),
                   mrope.apply(k, pos, SECTIONS[d], 1e4))
    s1 = np.einsum("ihd,jhd->hij", mrope.apply(q, pos + shift, SECTIONS[d], 1e4),
                   mrope.apply(k, pos + shift, SECTIONS[d], 1e4))
    assert np.abs(s0 - s1).max() < 1e-9


def test_norm_preserved_per_pair_and_identity_at_zero():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((10, 4, 64))
    pos = rng.uniform(0, 2e4, (10, 3)).astype(np.float32)
    y = mrope.apply(x, pos, SECTIONS[64], 1e4)
    nx = x[..., :32] ** 2 + x[..., 32:] ** 2
    ny = y[..., :32] ** 2 + y[..., 32:] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-12)
    np.testing.assert_array_equal(mrope.apply(x, np.zeros((10, 3), np.float32), SECTIONS[64], 1e4), x)


def test_axis_sections_touch_only_their_pairs():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 1, 128))
    st, sh, sw = SECTIONS[128]
    base = np.zeros((5, 3), np.float32)
    for axis, lo, hi in [(0, 0, st), (1, st, st + sh), (2, st + sh, st + sh + sw)]:
        pos = base.copy()
        pos[:, axis] = 3.0
        y = mrope.apply(x, pos, SECTIONS[128], 1e4)
        changed = ~np.isclose(y, x, rtol=0, atol=0)
        pairs = changed[..., :64] | changed[..., 64:]
        assert pairs[..., lo:hi].all()
        assert not pairs[..., :lo].any() and not pairs[..., hi:].any()


def test_rotation_direction_first_pair():
    # pair 0 has frequency 1: (1, 0) rotated by angle t is (cos t, sin t)
    x = np.zeros((1, 1, 64))
    x[0, 0, 0] = 1.0
    pos = np.array([[0.5, 0, 0]], np.float32)
    y = mrope.apply(x, pos, SECTIONS[64], 1e4)
    assert np.isclose(y[0, 0, 0], np.cos(0.5)) and np.isclose(y[0, 0, 32], np.sin(0.5))


def test_bad_sections_raise():
    with pytest.raises(ValueError):
        mrope.apply(np.zeros((1, 1, 64)), np.zeros((1, 3), np.float32), (8, 8, 8), 1e4)
