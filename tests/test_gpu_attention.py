"""GPU parity of mot_attention_fwd (both mask modes, fused mRoPE, LSE) and of
the mask / tile-class materialiser, against the fp64 oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as oattn
from oracle import layout as olayout
from oracle import mask as omask
from oracle import mrope as omrope
from tests.gpu_util import BF16_LSE_ATOL, assert_parity, device, say, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
AR, CH = W.AR_CAUSAL_DM_FULL, W.CHUNK_CAUSAL_KV


def _mot():
    import multimodal_diffusion_transformer_amd as mot
    return mot


def _qkv(seed, nq, nk, h, d, dtype, packed=True):
    """Seeded Q/K/V; with packed=True K/V are strided views of one
    [nk, 3, H, D] buffer (the projection's output layout)."""
    q = W.make(seed, W.T_Q, (nq, h, d), dtype)
    k = W.make(seed, W.T_K, (nk, h, d), dtype)
    v = W.make(seed, W.T_V, (nk, h, d), dtype)
    return q, k, v


def _to_dev(q, k, v, dev, packed):
    Q = W.to_torch(q, dev)
    if packed:
        nk, h, d = k.f32.shape
        buf = torch.empty((nk, 3, h, d), dtype=Q.dtype, device=dev)
        buf[:, 1].copy_(W.to_torch(k, dev))
        buf[:, 2].copy_(W.to_torch(v, dev))
        return Q, buf[:, 1], buf[:, 2]
    return Q, W.to_torch(k, dev), W.to_torch(v, dev)


CASES = [
    # name, nq, nk, q0, mode, n_ar, n_prefix, chunk_len, d
    ("ar_small_d128", 300, 300, 0, AR, 70, 0, 0, 128),
    ("ar_small_d64", 257, 257, 0, AR, 129, 0, 0, 64),
    ("ar_qoffset", 333, 1111, 700, AR, 514, 0, 0, 128),
    ("ar_all_causal", 190, 190, 0, AR, 190, 0, 0, 128),
    ("ar_no_text", 200, 200, 0, AR, 0, 0, 0, 128),
    ("ar_boundary_mid_tile", 1030, 1030, 0, AR, 514, 0, 0, 128),
    ("chunk_multi", 3 * 97 + 13, 258 + 3 * 97 + 13, 258, CH, 0, 258, 97, 128),
    ("chunk_small_chunks", 200, 230, 30, CH, 0, 30, 7, 64),
    ("chunk_no_prefix", 160, 160, 0, CH, 0, 0, 40, 128),
    ("single_query", 1, 5, 4, AR, 2, 0, 0, 128),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_parity_small(case):
    name, nq, nk, q0, mode, n_ar, n_prefix, chunk_len, d = case
    dev = device()
    mot = _mot()
    h = 4
    say("attention %s nq=%d nk=%d q0=%d d=%d" % (name, nq, nk, q0, d))
    q, k, v = _qkv(7, nq, nk, h, d, "bf16")
    Q, K, V = _to_dev(q, k, v, dev, packed=True)
    O = torch.empty((nq, h, d), dtype=torch.bfloat16, device=dev)
    L = torch.empty((h, nq), dtype=torch.float32, device=dev)
    mot.mot_attention_fwd(Q, K, V, O, mask=mode, q0=q0, n_ar=n_ar, n_prefix=n_prefix,
                          chunk_len=chunk_len, lse=L)
    torch.cuda.synchronize()
    want, lse = oattn.attention(q.f32, k.f32, v.f32, q0, mode, n_ar, n_prefix, max(chunk_len, 1))
    assert_parity(to_np(O), want, "bf16", name)
    np.testing.assert_allclose(to_np(L), lse, atol=BF16_LSE_ATOL, rtol=0)


def test_attention_fp32_tiny_workload_full():
    dev = device()
    mot = _mot()
    wl = W.BY_NAME["tiny_fp32"]
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h, d = len(reg), wl.n_heads, wl.head_dim
    q, k, v = _qkv(0, n, n, h, d, "fp32")
    Q, K, V = _to_dev(q, k, v, dev, packed=False)
    O = torch.empty((n, h, d), dtype=torch.float32, device=dev)
    mot.mot_attention_fwd(Q, K, V, O, mask=AR, n_ar=n_ar)
    torch.cuda.synchronize()
    want, _ = oattn.attention(q.f32, k.f32, v.f32, 0, AR, n_ar=n_ar)
    assert_parity(to_np(O), want, "fp32", "tiny fp32")


F32_CASES = [
    # name, nq, nk, q0, mode, n_ar, n_prefix, chunk_len, d
    ("f32_ar_d128", 150, 150, 0, AR, 40, 0, 0, 128),
    ("f32_ar_qoffset_d128", 70, 230, 160, AR, 100, 0, 0, 128),
    ("f32_chunk_d64", 3 * 37 + 5, 20 + 3 * 37 + 5, 20, CH, 0, 20, 37, 64),
    ("f32_chunk_d128", 2 * 45 + 7, 33 + 2 * 45 + 7, 33, CH, 0, 33, 45, 128),
]


@pytest.mark.parametrize("case", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_attention_fp32_parity(case):
    """The fp32 kernel at both head sizes and in both mask modes, with the
    LSE, against the oracle at the fp32 tolerance."""
    name, nq, nk, q0, mode, n_ar, n_prefix, chunk_len, d = case
    dev = device()
    mot = _mot()
    h = 3
    say("attention %s nq=%d nk=%d q0=%d d=%d" % (name, nq, nk, q0, d))
    q, k, v = _qkv(12, nq, nk, h, d, "fp32")
    Q, K, V = _to_dev(q, k, v, dev, packed=True)
    O = torch.empty((nq, h, d), dtype=torch.float32, device=dev)
    L = torch.empty((h, nq), dtype=torch.float32, device=dev)
    mot.mot_attention_fwd(Q, K, V, O, mask=mode, q0=q0, n_ar=n_ar, n_prefix=n_prefix,
                          chunk_len=chunk_len, lse=L)
    torch.cuda.synchronize()
    want, lse = oattn.attention(q.f32, k.f32, v.f32, q0, mode, n_ar, n_prefix, max(chunk_len, 1))
    assert_parity(to_np(O), want, "fp32", name)
    np.testing.assert_allclose(to_np(L), lse, atol=1e-4, rtol=0)


def test_attention_run_twice_is_bitwise_deterministic():
    """The same launch twice gives the same bits (no atomics, no order
    that depends on scheduling), for both kernels."""
    dev = device()
    mot = _mot()
    for dtype, n, d, n_ar in (("bf16", 1100, 128, 300), ("fp32", 200, 64, 70)):
        q, k, v = _qkv(13, n, n, 4, d, dtype)
        Q, K, V = _to_dev(q, k, v, dev, packed=True)
        outs = []
        for _ in range(2):
            O = torch.empty((n, 4, d), dtype=Q.dtype, device=dev)
            L = torch.empty((4, n), dtype=torch.float32, device=dev)
            mot.mot_attention_fwd(Q, K, V, O, mask=AR, n_ar=n_ar, lse=L)
            outs.append((O, L))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), dtype


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
@pytest.mark.parametrize("rope_k", [False, True])
def test_attention_fused_rope_on_load(dtype, d, rope_k):
    if rope_k and dtype == "bf16":
        pytest.skip("bf16 rotates Q on load only: the bf16 kernel variant that also rotated K on "
                    "load faulted the GPU (its tile copies read a base register that a vector "
                    "instruction had just written, with no wait states); the variant was removed "
                    "and the library rejects k_pos for bf16 (checked on the host)")
    dev = device()
    mot = _mot()
    wl = W.BY_NAME["policy_bf16"]
    pos, reg, n_ar = olayout.build(wl.segments)
    n = 700
    pos = pos[:n]
    n_ar = min(n_ar, n)
    h = 3
    secs = (d // 8, 3 * d // 16, 3 * d // 16)
    say("attention fused rope %s d=%d rope_k=%s" % (dtype, d, rope_k))
    q, k, v = _qkv(8, n, n, h, d, dtype)
    Q, K, V = _to_dev(q, k, v, dev, packed=True)
    Pd = torch.from_numpy(pos).to(dev)
    if not rope_k:
        mot.mrope_apply(K, Pd, secs, 1e4)
    O = torch.empty((n, h, d), dtype=Q.dtype, device=dev)
    mot.mot_attention_fwd(Q, K, V, O, mask=AR, n_ar=n_ar, q_pos=Pd,
                          k_pos=Pd if rope_k else None, sections=secs, theta=1e4)
    torch.cuda.synchronize()
    qr = omrope.apply(q.f32, pos, secs, 1e4)
    kr = omrope.apply(k.f32, pos, secs, 1e4)
    want, _ = oattn.attention(qr, kr, v.f32, 0, AR, n_ar=n_ar)
    assert_parity(to_np(O), want, "bf16" if dtype == "bf16" else "fp32", "fused rope")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("kind", ["jump", "first_tile_low"])
def test_attention_large_scores_move_the_reference(kind, d):
    """Scores far above the reference taken on a row's first tile (by 2^77
    and, for one key, past the fp32 range of exp2) and first tiles far below
    the rest: the kernel must move its softmax reference on the fly and
    still match the fp64 oracle."""
    dev = device()
    mot = _mot()
    nq = nk = 600
    n_ar, h = 100, 2
    say("attention large scores %s d=%d" % (kind, d))
    q, k, v = _qkv(11, nq, nk, h, d, "bf16")
    qf, kf = q.f32.copy(), k.f32.copy()
    if kind == "jump":
        qf[n_ar:, :, 0] += 8.0
        kf[300, :, 0] = 80.0    # ~2^81 above a random first tile's max
        kf[500, :, 0] = 150.0   # ~2^153: exp2 overflows without a new reference
    else:
        qf[n_ar:, :, 0] -= 8.0
        kf[:64, :, 0] = 80.0    # first tile ~2^-81 below the later ones
    qb = W.Tensor("bf16", W.bf16_bits(qf), W.bf16_to_f32(W.bf16_bits(qf)))
    kb = W.Tensor("bf16", W.bf16_bits(kf), W.bf16_to_f32(W.bf16_bits(kf)))
    Q, K, V = _to_dev(qb, kb, v, dev, packed=True)
    O = torch.empty((nq, h, d), dtype=torch.bfloat16, device=dev)
    L = torch.empty((h, nq), dtype=torch.float32, device=dev)
    mot.mot_attention_fwd(Q, K, V, O, mask=AR, n_ar=n_ar, lse=L)
    torch.cuda.synchronize()
    want, lse = oattn.attention(qb.f32, kb.f32, v.f32, 0, AR, n_ar=n_ar)
    assert_parity(to_np(O), want, "bf16", "large scores " + kind)
    # The row sum adds the bf16-rounded P that the PV product uses; here many
    # keys sit just below a row's max and their roundings share a sign
    # (BF16_LSE_ATOL).
    np.testing.assert_allclose(to_np(L), lse, atol=BF16_LSE_ATOL, rtol=0)


def test_attention_ar_rows_bitwise_invariant_to_dm():
    dev = device()
    mot = _mot()
    n, n_ar, h, d = 900, 300, 2, 128
    q, k, v = _qkv(9, n, n, h, d, "bf16")
    Q, K, V = _to_dev(q, k, v, dev, packed=False)
    O1 = torch.empty((n, h, d), dtype=torch.bfloat16, device=dev)
    O2 = torch.empty_like(O1)
    mot.mot_attention_fwd(Q, K, V, O1, mask=AR, n_ar=n_ar)
    Q2, K2, V2 = Q.clone(), K.clone(), V.clone()
    Q2[n_ar:] *= 2
    K2[n_ar:] = -K2[n_ar:]
    V2[n_ar:] += 3
    mot.mot_attention_fwd(Q2, K2, V2, O2, mask=AR, n_ar=n_ar)
    torch.cuda.synchronize()
    a, b = O1.cpu().view(torch.int16), O2.cpu().view(torch.int16)
    assert torch.equal(a[:n_ar], b[:n_ar])
    assert not torch.equal(a[n_ar:], b[n_ar:])


def test_attention_chunk_rows_bitwise_invariant_to_future_chunks():
    dev = device()
    mot = _mot()
    n_prefix, c, h, d = 64, 150, 2, 128
    nq = 3 * c
    nk = n_prefix + nq
    q, k, v = _qkv(10, nq, nk, h, d, "bf16")
    Q, K, V = _to_dev(q, k, v, dev, packed=False)
    O1 = torch.empty((nq, h, d), dtype=torch.bfloat16, device=dev)
    O2 = torch.empty_like(O1)
    kw = dict(mask=CH, q0=n_prefix, n_prefix=n_prefix, chunk_len=c)
    mot.mot_attention_fwd(Q, K, V, O1, **kw)
    K2, V2 = K.clone(), V.clone()
    K2[n_prefix + c:] *= -1
    V2[n_prefix + c:] -= 2
    mot.mot_attention_fwd(Q, K2, V2, O2, **kw)
    torch.cuda.synchronize()
    a, b = O1.cpu().view(torch.int16), O2.cpu().view(torch.int16)
    assert torch.equal(a[:c], b[:c])
    assert not torch.equal(a[c:], b[c:])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_attention_with_no_query_rows_is_a_no_op(dtype):
    """An empty query block (and an empty LSE) through the binding: the
    call returns and writes nothing."""
    dev = device()
    mot = _mot()
    h, d, nk = 2, 128, 70
    k = torch.ones((nk, h, d), dtype=dtype, device=dev)
    q = torch.empty((0, h, d), dtype=dtype, device=dev)
    o = torch.empty((0, h, d), dtype=dtype, device=dev)
    lse = torch.empty((h, 0), dtype=torch.float32, device=dev)
    guard = torch.full((4,), 7.0, device=dev)
    mot.mot_attention_fwd(q, k, k, o, mask=mot.MOT_AR_CAUSAL_DM_FULL, n_ar=10, lse=lse)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(guard, torch.full((4,), 7.0, device=dev))


def test_attention_first_row_is_first_value_exactly():
    dev = device()
    mot = _mot()
    n, h, d = 300, 2, 128
    q, k, v = _qkv(11, n, n, h, d, "bf16")
    Q, K, V = _to_dev(q, k, v, dev, packed=False)
    O = torch.empty((n, h, d), dtype=torch.bfloat16, device=dev)
    mot.mot_attention_fwd(Q, K, V, O, mask=AR, n_ar=100)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(O)[0], v.f32[0])


@pytest.mark.parametrize("case", [
    dict(nq=1030, nk=1030, q0=0, mask=AR, n_ar=514),
    dict(nq=333, nk=1111, q0=700, mask=AR, n_ar=514),
    dict(nq=3 * 97 + 13, nk=258 + 3 * 97 + 13, q0=258, mask=CH, n_prefix=258, chunk_len=97),
])
def test_mask_and_tile_materialiser_exact(case):
    dev = device()
    mot = _mot()
    a = mot.mask_args(**case)
    nq, nk = case["nq"], case["nk"]
    M = torch.empty((nq, nk), dtype=torch.uint8, device=dev)
    bm, bn = 128, 64
    T = torch.empty((-(-nq // bm), -(-nk // bn)), dtype=torch.uint8, device=dev)
    mot.mot_mask_materialize(a, M, bm, bn, T)
    torch.cuda.synchronize()
    want = omask.materialize(nq, nk, case["q0"], case["mask"], case.get("n_ar", 0),
                             case.get("n_prefix", 0), case.get("chunk_len", 1))
    np.testing.assert_array_equal(M.cpu().numpy().astype(bool), want)
    np.testing.assert_array_equal(T.cpu().numpy(), omask.tile_classes(want, bm, bn))


def test_attention_policy_workload_full():
    dev = device()
    mot = _mot()
    wl = W.BY_NAME["policy_bf16"]
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h, d = len(reg), wl.n_heads, wl.head_dim
    say("attention policy workload full n=%d" % n)
    q, k, v = _qkv(wl.wid, n, n, h, d, "bf16")
    Q, K, V = _to_dev(q, k, v, dev, packed=True)
    O = torch.empty((n, h, d), dtype=torch.bfloat16, device=dev)
    mot.mot_attention_fwd(Q, K, V, O, mask=AR, n_ar=n_ar)
    torch.cuda.synchronize()
    want, _ = oattn.attention(q.f32, k.f32, v.f32, 0, AR, n_ar=n_ar)
    assert_parity(to_np(O), want, "bf16", "policy full")


def _sample_rows(n, n_ar, rng, extra=48):
    rows = set(range(min(n_ar + 2, n)))  # all AR rows and the boundary
    rows |= {n - 1, n - 2}
    rows |= set(int(r) for r in rng.choice(n, size=min(extra, n), replace=False))
    return sorted(rows)


@pytest.mark.parametrize("name", ["t2v480p_bf16", "t2v480p_long_bf16"])
def test_attention_long_workloads_sampled_rows(name):
    dev = device()
    mot = _mot()
    wl = W.BY_NAME[name]
    n = wl.n_tokens
    n_ar = W.region_counts(wl.segments)[0]
    h, d = wl.n_heads, wl.head_dim
    say("attention %s sampled rows n=%d" % (name, n))
    q, k, v = _qkv(wl.wid, n, n, h, d, "bf16")
    Q, K, V = _to_dev(q, k, v, dev, packed=True)
    O = torch.empty((n, h, d), dtype=torch.bfloat16, device=dev)
    mot.mot_attention_fwd(Q, K, V, O, mask=AR, n_ar=n_ar)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = _sample_rows(n, n_ar, rng, extra=32)
    heads = [0, 7, 23] if len(rows) > 100 else list(range(h))
    want = oattn.attention_rows(q.f32[rows], k.f32, v.f32, rows, heads, 0, AR, n_ar=n_ar)
    got = to_np(O)[rows][:, heads]
    assert_parity(got, want, "bf16", name + " sampled")
