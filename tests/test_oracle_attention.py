"""Pins of the oracle's masked attention (CPU only)."""
import numpy as np
import pytest

import workloads as W
from oracle import attention, layout, mask

AR, CH = W.AR_CAUSAL_DM_FULL, W.CHUNK_CAUSAL_KV


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("case", [
    dict(nq=9, nk=9, q0=0, mode=AR, n_ar=4),
    dict(nq=6, nk=11, q0=5, mode=AR, n_ar=7),
    dict(nq=7, nk=12, q0=5, mode=CH, n_prefix=3, chunk_len=2),
    dict(nq=4, nk=10, q0=6, mode=CH, n_prefix=6, chunk_len=4),
])
def test_vectorised_equals_bruteforce(case):
    nq, nk, q0, mode = case["nq"], case["nk"], case["q0"], case["mode"]
    kw = {k: v for k, v in case.items() if k in ("n_ar", "n_prefix", "chunk_len")}
    h, d = 2, 8
    q, k, v = _rand((nq, h, d), 1), _rand((nk, h, d), 2), _rand((nk, h, d), 3)
    o1, l1 = attention.attention(q, k, v, q0, mode, row_block=3, **kw)
    o2, l2 = attention.attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), q0, mode, **kw)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_tiny_workload_bruteforce_sampled_rows():
    wl = W.BY_NAME["tiny_fp32"]
    n = wl.n_tokens
    n_ar = W.region_counts(wl.segments)[0]
    q = W.make(0, W.T_Q, (n, 4, 64), "fp32").f32
    k = W.make(0, W.T_K, (n, 4, 64), "fp32").f32
    v = W.make(0, W.T_V, (n, 4, 64), "fp32").f32
    o, _ = attention.attention(q, k, v, 0, AR, n_ar=n_ar)
    rows = [0, 1, 33, 34, 60, 113]
    # brute force one row at a time, at its absolute index
    for r in rows:
        orow, _ = attention.attention_bruteforce(q[r:r + 1].tolist(), k.tolist(), v.tolist(), r, AR, n_ar=n_ar)
        np.testing.assert_allclose(o[r], orow[0], rtol=0, atol=1e-12)


def test_first_row_reads_only_first_key():
    q, k, v = _rand((8, 3, 16), 4), _rand((8, 3, 16), 5), _rand((8, 3, 16), 6)
    o, lse = attention.attention(q, k, v, 0, AR, n_ar=5)
    np.testing.assert_array_equal(o[0], v[0])


def test_zero_query_gives_mean_of_allowed_values():
    n, n_ar = 12, 5
    q = np.zeros((n, 2, 8))
    k, v = _rand((n, 2, 8), 7), _rand((n, 2, 8), 8)
    o, lse = attention.attention(q, k, v, 0, AR, n_ar=n_ar)
    for i in range(n):
        keys = np.arange(i + 1) if i < n_ar else np.arange(n)
        np.testing.assert_allclose(o[i], v[keys].mean(axis=0), atol=1e-13)
        np.testing.assert_allclose(lse[:, i], np.log(len(keys)), atol=1e-13)


def test_dm_outputs_invariant_to_dm_key_permutation():
    n, n_ar = 20, 6
    q, k, v = _rand((n, 2, 8), 9), _rand((n, 2, 8), 10), _rand((n, 2, 8), 11)
    o, _ = attention.attention(q, k, v, 0, AR, n_ar=n_ar)
    perm = np.concatenate([np.arange(n_ar), n_ar + np.random.default_rng(0).permutation(n - n_ar)])
    # permute the DM keys/values only; queries stay in place
    o2, _ = attention.attention(q, k[perm], v[perm], 0, AR, n_ar=n_ar)
    np.testing.assert_allclose(o2[n_ar:], o[n_ar:], atol=1e-13)


def test_ar_rows_bitwise_invariant_to_dm_perturbation():
    n, n_ar = 300, 40
    q, k, v = _rand((n, 2, 16), 12), _rand((n, 2, 16), 13), _rand((n, 2, 16), 14)
    o, l = attention.attention(q, k, v, 0, AR, n_ar=n_ar)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[n_ar:] += 5
    k2[n_ar:] *= -3
    v2[n_ar:] += 100
    o2, l2 = attention.attention(q2, k2, v2, 0, AR, n_ar=n_ar)
    np.testing.assert_array_equal(o2[:n_ar], o[:n_ar])
    np.testing.assert_array_equal(l2[:, :n_ar], l[:, :n_ar])
    assert not np.allclose(o2[n_ar:], o[n_ar:])


def test_chunk_rows_invariant_to_future_chunks():
    n_prefix, c = 5, 6
    nk = n_prefix + 4 * c
    q = _rand((4 * c, 2, 8), 15)
    k, v = _rand((nk, 2, 8), 16), _rand((nk, 2, 8), 17)
    o, _ = attention.attention(q, k, v, n_prefix, CH, n_prefix=n_prefix, chunk_len=c)
    for ch in range(3):
        cut = n_prefix + (ch + 1) * c
        k2, v2, q2 = k.copy(), v.copy(), q.copy()
        k2[cut:] += 3
        v2[cut:] -= 7
        q2[(ch + 1) * c:] *= 2
        o2, _ = attention.attention(q2, k2, v2, n_prefix, CH, n_prefix=n_prefix, chunk_len=c)
        np.testing.assert_array_equal(o2[:(ch + 1) * c], o[:(ch + 1) * c])


def test_rows_helper_matches_full():
    n, n_ar = 50, 9
    q, k, v = _rand((n, 3, 8), 18), _rand((n, 3, 8), 19), _rand((n, 3, 8), 20)
    o, _ = attention.attention(q, k, v, 0, AR, n_ar=n_ar)
    rows = [0, 8, 9, 49]
    heads = [0, 2]
    orow = attention.attention_rows(q[rows], k, v, rows, heads, 0, AR, n_ar=n_ar)
    np.testing.assert_allclose(orow, o[rows][:, heads], atol=1e-13)


def test_flop_count_definition():
    assert attention.flops(635963395, 24, 128) == pytest.approx(7.815e12, rel=1e-3)


def test_single_key_row_lse_is_its_score():
    """Row 0 of the AR-causal mask sees key 0 alone: LSE = q0.k0 * scale."""
    q, k, v = _rand((6, 2, 16), 11), _rand((6, 2, 16), 12), _rand((6, 2, 16), 13)
    _, lse = attention.attention(q, k, v, 0, AR, n_ar=4)
    want = (q[0] * k[0]).sum(axis=1) / 4.0  # scale = 1/sqrt(16)
    np.testing.assert_allclose(lse[:, 0], want, rtol=0, atol=1e-14)


def test_two_key_row_is_a_logistic_mix():
    """Row 1 of the AR-causal mask sees keys 0 and 1: the softmax reduces to a
    logistic weight w = 1 / (1 + exp(s1 - s0)) and LSE = s0 + log1p(exp(s1 - s0))."""
    q, k, v = _rand((5, 3, 8), 21), _rand((5, 3, 8), 22), _rand((5, 3, 8), 23)
    o, lse = attention.attention(q, k, v, 0, AR, n_ar=5)
    sc = 1.0 / np.sqrt(8.0)
    for h in range(3):
        s0 = float(q[1, h] @ k[0, h]) * sc
        s1 = float(q[1, h] @ k[1, h]) * sc
        w0 = 1.0 / (1.0 + np.exp(s1 - s0))
        np.testing.assert_allclose(o[1, h], w0 * v[0, h] + (1.0 - w0) * v[1, h], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[h, 1], s0 + np.log1p(np.exp(s1 - s0)), rtol=0, atol=1e-13)


def test_huge_scores_stay_finite():
    """Scores of +-1e3 (far past exp's range) must go through the max
    subtraction: O is the value of the dominant key and LSE its score."""
    d = 4
    q = np.zeros((3, 1, d)); q[:, 0, 0] = 1.0
    k = np.zeros((3, 1, d)); k[:, 0, 0] = [0.0, 2000.0, -2000.0]
    v = _rand((3, 1, d), 31)
    o, lse = attention.attention(q, k, v, 0, AR, n_ar=0)  # all DM: every row sees all keys
    for i in range(3):
        np.testing.assert_allclose(o[i, 0], v[1, 0], rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[0, i], 1000.0, rtol=0, atol=1e-12)  # 2000 * 1/sqrt(4)


def test_merge_of_key_partitions_is_attention_over_all_keys():
    # softmax attention over a union of key sets from the parts' outputs and
    # log-sum-exps: the identity a key-split launch relies on
    rng = np.random.default_rng(71)
    nq, nk, h, d = 9, 40, 3, 8
    q, k, v = rng.standard_normal((nq, h, d)), rng.standard_normal((nk, h, d)), rng.standard_normal((nk, h, d))
    full, lse_full = attention.attention(q, k, v, nk, W.AR_CAUSAL_DM_FULL, n_ar=0)
    for cuts in ([20], [7, 25], [1], [39]):
        edges = [0] + cuts + [nk]
        parts = [attention.attention(q, k[a:b], v[a:b], b - a, W.AR_CAUSAL_DM_FULL, n_ar=0)
                 for a, b in zip(edges[:-1], edges[1:])]
        o, lse = attention.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        np.testing.assert_allclose(o, full, atol=1e-13)
        np.testing.assert_allclose(lse, lse_full, atol=1e-13)


def test_merge_single_part_and_empty_part():
    rng = np.random.default_rng(72)
    o1, l1 = rng.standard_normal((1, 4, 2, 8)), rng.standard_normal((1, 2, 4))
    o, l = attention.merge(o1, l1)
    np.testing.assert_allclose(o, o1[0], atol=1e-15)
    np.testing.assert_allclose(l, l1[0], atol=1e-15)
    # a part with no keys (LSE = -inf) has weight 0
    o2 = np.concatenate([o1, rng.standard_normal((1, 4, 2, 8))])
    l2 = np.concatenate([l1, np.full((1, 2, 4), -np.inf)])
    o, l = attention.merge(o2, l2)
    np.testing.assert_allclose(o, o1[0], atol=1e-15)
