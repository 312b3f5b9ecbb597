"""Pins of the oracle's masks and tile classes (CPU only)."""
import numpy as np
import pytest

import workloads as W
from oracle import mask


def _block_form_ar_dm(n_ar, n):
    """The two equations of the joint attention written as blocks:
    O_AR = causal attention inside AR (lower triangle, no DM columns);
    O_DM = full attention over [K_AR; K_DM] (all ones)."""
    m = np.zeros((n, n), dtype=bool)
    m[:n_ar, :n_ar] = np.tril(np.ones((n_ar, n_ar), dtype=bool))
    m[n_ar:, :] = True
    return m


@pytest.mark.parametrize("n_ar,n", [(1, 1), (3, 6), (34, 114), (7, 40), (40, 40)])
def test_ar_dm_mask_equals_block_form(n_ar, n):
    np.testing.assert_array_equal(
        mask.materialize(n, n, 0, W.AR_CAUSAL_DM_FULL, n_ar=n_ar),
        _block_form_ar_dm(n_ar, n))


def test_ar_dm_mask_with_query_offset():
    full = _block_form_ar_dm(9, 30)
    np.testing.assert_array_equal(
        mask.materialize(12, 30, 9, W.AR_CAUSAL_DM_FULL, n_ar=9), full[9:21])


def test_chunk_mask_block_form():
    n_prefix, c, nch = 5, 4, 3
    n = n_prefix + c * nch + 2          # ragged last chunk of 2
    chunks = nch + 1
    want = np.zeros((n, n), dtype=bool)
    want[:, :n_prefix] = True
    blocks = np.kron(np.tril(np.ones((chunks, chunks), dtype=bool)),
                     np.ones((c, c), dtype=bool))[: n - n_prefix, : n - n_prefix]
    want[n_prefix:, n_prefix:] = blocks
    got = mask.materialize(n - n_prefix, n, n_prefix, W.CHUNK_CAUSAL_KV,
                           n_prefix=n_prefix, chunk_len=c)
    np.testing.assert_array_equal(got, want[n_prefix:])


def test_tile_classes_hand_example():
    m = mask.materialize(6, 6, 0, W.AR_CAUSAL_DM_FULL, n_ar=3)
    E, P, F = mask.EMPTY, mask.PARTIAL, mask.FULL
    want = np.array([[P, E, E], [F, P, P], [F, F, F]], dtype=np.uint8)
    np.testing.assert_array_equal(mask.tile_classes(m, 2, 2), want)


def test_tile_classes_ragged_edges():
    m = mask.materialize(5, 7, 0, W.AR_CAUSAL_DM_FULL, n_ar=5)
    tc = mask.tile_classes(m, 4, 4)
    # rows 0-3 x cols 0-3: lower triangle -> partial; rows 0-3 x cols 4-6:
    # empty; row 4 x cols 0-3: full; row 4 x cols 4-6: only (4,4) -> partial
    np.testing.assert_array_equal(tc, [[mask.PARTIAL, mask.EMPTY],
                                       [mask.FULL, mask.PARTIAL]])


@pytest.mark.parametrize("wl", [w for w in W.WORKLOADS if w.mask == W.AR_CAUSAL_DM_FULL],
                         ids=lambda w: w.name)
def test_pair_count_closed_form(wl):
    n = wl.n_tokens
    n_ar = W.region_counts(wl.segments)[0]
    closed = n_ar * (n_ar + 1) // 2 + (n - n_ar) * n
    if n <= 4000:
        assert mask.count_pairs(n, n, 0, W.AR_CAUSAL_DM_FULL, n_ar=n_ar) == closed
    else:
        # count a window of rows around the boundary and extrapolate the
        # DM rows, which all see every key
        got = mask.count_pairs(n_ar + 64, n, 0, W.AR_CAUSAL_DM_FULL, n_ar=n_ar)
        assert got + (n - n_ar - 64) * n == closed


def test_chunk_pair_count_closed_form():
    n_prefix, c = 258, 1440
    nk = n_prefix + 9 * c
    got = mask.count_pairs(c, nk, n_prefix + 8 * c, W.CHUNK_CAUSAL_KV,
                           n_prefix=n_prefix, chunk_len=c)
    assert got == c * nk == 19033920
    got = mask.count_pairs(3 * c, n_prefix + 3 * c, n_prefix, W.CHUNK_CAUSAL_KV,
                           n_prefix=n_prefix, chunk_len=c)
    assert got == sum(c * (n_prefix + (k + 1) * c) for k in range(3))
