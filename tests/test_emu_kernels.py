"""The library's kernels, run on the CPU SIMT emulator, against the oracle.

tests/emu_lib.py compiles the product kernel sources (csrc/*.hip, with only
their inline-asm lines swapped for the emulator's equivalents) for the host;
tests/native/emu runs every work-item as a fiber and performs the wave and
workgroup operations (MFMA, transposing LDS reads, LDS-DMA copies, lane
swaps, ballots, barriers) with their CDNA4 semantics.  The same C entry
points the GPU tests call are called here on guarded host buffers, at the
same tolerances, so the index arithmetic, masking, tile schedules, GQA
head mapping, batching, epilogues and reductions of each kernel are checked
with no GPU.  Two run modes cover scheduling: LDS-DMA copies landing at once
with waves run in order, and copies held back until the issuing wave's
vmcnt wait (their LDS slots reading NaN meanwhile) with waves run in
reverse; a third, a seeded random wave order in every phase between
barriers, is drawn by tests/test_emu_fuzz.py and by the check that results
are the same bits in every mode.  A planted mistake in a copy of the sources (a missing wait, a
missing barrier, a wrong key/value head, an unclamped ragged tile) must make
these checks fail.

What the emulator cannot show: timing, hazards between instructions (the
disassembly scans cover those), and register allocation.
"""
import ctypes
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import attention as oattn
from oracle import block as oblock
from oracle import cfg as ocfg
from oracle import euler as oeuler
from oracle import layout as olayout
from oracle import mrope as omrope
from oracle import projection as oproj
from tests import emu_lib
from tests.gpu_util import BF16_LSE_ATOL, assert_parity, assert_parity_stored, errors

pytestmark = pytest.mark.skipif(not os.path.exists(emu_lib.CXX), reason="host clang++ missing")
# the C ABI's argument structure and types, as the product binding declares them
mot_attn_args = pytest.importorskip("multimodal_diffusion_transformer_amd._binding").mot_attn_args

AR, CH = W.AR_CAUSAL_DM_FULL, W.CHUNK_CAUSAL_KV
BF16, FP32 = 0, 1
MODES = [(False, False), (True, True)]  # (copies held until the wait, waves in reverse)
MODE_IDS = ["dma_early_fwd", "dma_late_rev"]


@pytest.fixture(scope="module")
def lib_path(tmp_path_factory):
    return emu_lib.build(str(tmp_path_factory.mktemp("emu")))


@pytest.fixture(scope="module")
def E(lib_path):
    e = emu_lib.Emu(lib_path)
    yield e
    e.free_all()


@pytest.fixture(autouse=True)
def _free(request):
    yield
    if "E" in request.fixturenames:
        request.getfixturevalue("E").free_all()


def _el(t):
    return [s // t.itemsize for s in t.strides]


def bits_of(x):
    return W.bf16_bits(np.asarray(x, np.float32))


def val(bits):
    return W.bf16_to_f32(np.asarray(bits))


# ---------------------------------------------------------------------------
# attention
def attn_args(q, k, v, o, *, mode, q0=0, n_ar=0, n_prefix=0, chunk_len=0, lse=None, q_pos=None,
              k_pos=None, sections=(0, 0, 0), theta=1e4, scale=0.0):
    """mot_attn_args for [N, H, D] arrays, or [B, N, H, D] with the batch
    stride taken from dimension 0 (0 shares one tensor)."""
    batched = q.ndim == 4
    a = mot_attn_args()
    a.q, a.k, a.v, a.o = q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data
    a.lse = None if lse is None else lse.ctypes.data
    a.dt = BF16 if q.dtype == np.uint16 else FP32
    sq, sk, sv, so = (_el(t) for t in (q, k, v, o))
    if batched:
        a.n_batch = q.shape[0]
        a.q_bs, a.k_bs, a.v_bs, a.o_bs = sq[0], sk[0], sv[0], so[0]
        sq, sk, sv, so = sq[1:], sk[1:], sv[1:], so[1:]
    nq, h, d = q.shape[-3:]
    a.n_heads, a.head_dim, a.mask = h, d, mode
    a.nq, a.nk, a.q0 = nq, k.shape[-3], q0
    a.q_ts, a.q_hs, a.k_ts, a.k_hs = sq[0], sq[1], sk[0], sk[1]
    a.v_ts, a.v_hs, a.o_ts, a.o_hs = sv[0], sv[1], so[0], so[1]
    a.n_ar, a.n_prefix, a.chunk_len = n_ar, n_prefix, chunk_len
    a.q_pos = None if q_pos is None else q_pos.ctypes.data
    a.k_pos = None if k_pos is None else k_pos.ctypes.data
    a.sec_t, a.sec_h, a.sec_w = sections
    a.theta, a.scale = theta, scale
    a.n_kv_heads = k.shape[-2]
    return a


def attention(E, q, k, v, o, **kw):
    st = E.call("mot_attention_fwd", ctypes.byref(attn_args(q, k, v, o, **kw)), None)
    assert st == 0, st


CASES = [
    # name, nq, nk, q0, mode, n_ar, n_prefix, chunk_len, d, H, H_kv
    ("ar_small_d128", 300, 300, 0, AR, 70, 0, 0, 128, 4, 4),
    ("ar_small_d64", 257, 257, 0, AR, 129, 0, 0, 64, 4, 4),
    ("ar_qoffset", 333, 1111, 700, AR, 514, 0, 0, 128, 2, 2),
    ("ar_all_causal", 190, 190, 0, AR, 190, 0, 0, 128, 2, 2),
    ("ar_no_text", 200, 200, 0, AR, 0, 0, 0, 64, 2, 2),
    ("ar_boundary_mid_tile", 600, 600, 0, AR, 258, 0, 0, 128, 2, 2),
    ("chunk_multi", 3 * 97 + 13, 258 + 3 * 97 + 13, 258, CH, 0, 258, 97, 128, 2, 2),
    ("chunk_small_chunks", 200, 230, 30, CH, 0, 30, 7, 64, 2, 2),
    ("chunk_no_prefix", 160, 160, 0, CH, 0, 0, 40, 128, 2, 2),
    ("single_query", 1, 5, 4, AR, 2, 0, 0, 128, 2, 2),
    ("gqa_2to1_d128", 300, 300, 0, AR, 70, 0, 0, 128, 4, 2),
    ("gqa_8_per_kv_d64", 130, 200, 70, AR, 90, 0, 0, 64, 8, 1),
    ("gqa_16_4_xcd_map", 140, 140, 0, AR, 50, 0, 0, 64, 16, 4),
    ("nano_heads_32_8", 100, 100, 0, AR, 30, 0, 0, 128, 32, 8),
    ("gqa_chunk", 2 * 64 + 9, 40 + 2 * 64 + 9, 40, CH, 0, 40, 64, 128, 8, 2),
    ("ar_small_d80", 300, 300, 0, AR, 70, 0, 0, 80, 4, 4),
    ("ar_qoffset_d80", 150, 333, 183, AR, 100, 0, 0, 80, 2, 2),
    ("chunk_d80", 2 * 64 + 9, 40 + 2 * 64 + 9, 40, CH, 0, 40, 64, 80, 4, 2),
    ("super_heads_64_8_d80", 100, 100, 0, AR, 30, 0, 0, 80, 64, 8),
]


def _qkv(seed, nq, nk, h, hk, d, dt):
    q = W.make(seed, W.T_Q, (nq, h, d), dt)
    k = W.make(seed, W.T_K, (nk, hk, d), dt)
    v = W.make(seed, W.T_V, (nk, hk, d), dt)
    return q, k, v


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_bf16(E, case, mode):
    name, nq, nk, q0, mask, n_ar, n_prefix, cl, d, h, hk = case
    E.config(*mode)
    q, k, v = _qkv(7, nq, nk, h, hk, d, "bf16")
    Q, K, V = E.array(q.bits), E.array(k.bits), E.array(v.bits)
    O, L = E.empty((nq, h, d), np.uint16), E.empty((h, nq), np.float32)
    attention(E, Q, K, V, O, mode=mask, q0=q0, n_ar=n_ar, n_prefix=n_prefix, chunk_len=cl, lse=L)
    want, lse = oattn.attention(q.f32, k.f32, v.f32, q0, mask, n_ar, n_prefix, max(cl, 1))
    assert_parity(val(O), want, "bf16", name)
    np.testing.assert_allclose(L, lse, atol=BF16_LSE_ATOL, rtol=0)


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("mask", [AR, CH], ids=["ar", "chunk"])
def test_attention_d80_is_d128_on_zero_padded_heads(E, mode, mask):
    """At the same scale (1/sqrt(80)), the D = 80 kernel and the D = 128
    kernel given the same heads zero-padded to 128 dims compute the same
    scores, the same P and the same dims 0..79 of O: bitwise equal O and
    LSE."""
    E.config(*mode)
    nq, nk, q0, h, hk = 150, 333, 183, 8, 2
    kw = dict(n_ar=100) if mask == AR else dict(n_prefix=40, chunk_len=70)
    q, k, v = _qkv(60, nq, nk, h, hk, 80, "bf16")
    outs = []
    for d in (80, 128):
        pad = lambda t: np.pad(t.bits, ((0, 0), (0, 0), (0, d - 80)))
        O, L = E.empty((nq, h, d), np.uint16), E.empty((h, nq), np.float32)
        attention(E, E.array(pad(q)), E.array(pad(k)), E.array(pad(v)), O, mode=mask, q0=q0, lse=L,
                  scale=1.0 / math.sqrt(80.0), **kw)
        outs.append((np.array(O[..., :80]), np.array(L)))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    want, _ = oattn.attention(q.f32, k.f32, v.f32, q0, mask, **{**kw, "chunk_len": kw.get("chunk_len", 1)})
    assert_parity(val(outs[0][0]), want, "bf16", "D = 80")


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_attention_bf16_strided_packed_views(E, mode):
    """K and V as strided views of one [nk, 3, H, D] buffer (the projection's
    output layout) and Q, O with padded rows."""
    E.config(*mode)
    nq, h, d, n_ar = 333, 4, 128, 120
    q, k, v = _qkv(8, nq, nq, h, h, d, "bf16")
    buf = E.empty((nq, 3, h, d), np.uint16)
    buf[:, 1], buf[:, 2] = k.bits, v.bits
    Qp = E.empty((nq, h + 1, d), np.uint16)
    Qp[:, :h] = q.bits
    Op = E.empty((nq, h + 1, d), np.uint16)
    attention(E, Qp[:, :h], buf[:, 1], buf[:, 2], Op[:, :h], mode=AR, n_ar=n_ar)
    want, _ = oattn.attention(q.f32, k.f32, v.f32, 0, AR, n_ar)
    assert_parity(val(Op[:, :h]), want, "bf16", "strided")
    assert (Op[:, h] == 0).all()  # the pad head is never written


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("d", [128, 64, 80])
def test_attention_bf16_batched_heads_and_strides(E, mode, d):
    """Two batch items with their own Q, K, V, O, LSE (GQA 4 -> 2), against
    the oracle per item."""
    E.config(*mode)
    B, nq, h, hk, n_ar = 2, 210, 4, 2, 80
    Q = E.empty((B, nq, h, d), np.uint16)
    K = E.empty((B, nq, hk, d), np.uint16)
    V = E.empty((B, nq, hk, d), np.uint16)
    ins = []
    for b in range(B):
        q, k, v = _qkv(20 + b, nq, nq, h, hk, d, "bf16")
        Q[b], K[b], V[b] = q.bits, k.bits, v.bits
        ins.append((q, k, v))
    O, L = E.empty((B, nq, h, d), np.uint16), E.empty((B, h, nq), np.float32)
    attention(E, Q, K, V, O, mode=AR, n_ar=n_ar, lse=L)
    for b, (q, k, v) in enumerate(ins):
        want, lse = oattn.attention(q.f32, k.f32, v.f32, 0, AR, n_ar)
        assert_parity(val(O[b]), want, "bf16", "batch item %d" % b)
        np.testing.assert_allclose(L[b], lse, atol=BF16_LSE_ATOL, rtol=0)


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_attention_key_split_and_merge(E, mode):
    """The streaming call's key split: one batched launch over two
    overlapping views of one K/V cache (batch stride = half the keys, Q
    shared with batch stride 0), then mot_attention_merge, equals attention
    over all keys."""
    E.config(*mode)
    nq, half, h, d = 150, 200, 4, 128
    q, k, v = _qkv(30, nq, 2 * half, h, h, d, "bf16")
    Q, K, V = E.array(q.bits), E.array(k.bits), E.array(v.bits)
    st = np.lib.stride_tricks
    Qb = st.as_strided(Q, (2, nq, h, d), (0,) + Q.strides)
    Kb = st.as_strided(K, (2, half, h, d), (half * K.strides[0],) + K.strides)
    Vb = st.as_strided(V, (2, half, h, d), (half * V.strides[0],) + V.strides)
    Op, Lp = E.empty((2, nq, h, d), np.uint16), E.empty((2, h, nq), np.float32)
    attention(E, Qb, Kb, Vb, Op, mode=AR, n_ar=0, lse=Lp)
    O, L = E.empty((nq, h, d), np.uint16), E.empty((h, nq), np.float32)
    el = _el(Op)
    st_ = E.call("mot_attention_merge", emu_lib.ptr(Op), emu_lib.ptr(Lp), 2, el[0], nq, h, d, el[1], el[2],
                 emu_lib.ptr(O), h * d, d, emu_lib.ptr(L), BF16, None)
    assert st_ == 0
    want, lse = oattn.attention(q.f32, k.f32, v.f32, 0, AR, n_ar=0)
    assert_parity(val(O), want, "bf16", "split + merge")
    np.testing.assert_allclose(L, lse, atol=BF16_LSE_ATOL, rtol=0)


@pytest.mark.parametrize("d", [128, 64, 80])
def test_attention_bf16_rope_q_on_load(E, d):
    E.config(True, True)
    wl = W.BY_NAME["policy_bf16"]
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h = 300, 2
    pos = np.ascontiguousarray(pos[:n])
    n_ar = min(n_ar, n)
    secs = (d // 8, 3 * d // 16, 3 * d // 16)
    q, k, v = _qkv(8, n, n, h, h, d, "bf16")
    kr = omrope.apply(k.f32, pos, secs, 1e4)
    kb = bits_of(kr)
    Q, K, V, P = E.array(q.bits), E.array(kb), E.array(v.bits), E.array(pos)
    O = E.empty((n, h, d), np.uint16)
    attention(E, Q, K, V, O, mode=AR, n_ar=n_ar, q_pos=P, sections=secs, theta=1e4)
    qr = omrope.apply(q.f32, pos, secs, 1e4)
    want, _ = oattn.attention(qr, val(kb), v.f32, 0, AR, n_ar=n_ar)
    assert_parity(val(O), want, "bf16", "rope on load")


@pytest.mark.parametrize("kind,hk,d", [("jump", 2, 128), ("jump", 1, 128), ("first_tile_low", 2, 128),
                                        ("first_tile_low", 1, 128), ("jump", 1, 80), ("first_tile_low", 2, 80)])
def test_attention_large_scores_move_the_reference(E, kind, hk, d):
    """The rare path that recomputes a tile's scores from K in global memory
    (overflow of the tile sum past 2^64), with GQA and a second batch item so
    that its K addressing uses both; at D = 80 its k-step count is odd."""
    E.config(True, True)
    nq, n_ar, h = 400, 100, 2
    Qs, Ks, Vs, ins = [], [], [], []
    for b in range(2):
        q, k, v = _qkv(11 + b, nq, nq, h, hk, d, "bf16")
        qf, kf = q.f32.copy(), k.f32.copy()
        if kind == "jump":
            qf[n_ar:, :, 0] += 8.0
            kf[300, :, 0] = 80.0
            kf[350, :, 0] = 150.0
        else:
            qf[n_ar:, :, 0] -= 8.0
            kf[:64, :, 0] = 80.0
        ins.append((val(bits_of(qf)), val(bits_of(kf)), v.f32))
        Qs.append(bits_of(qf)), Ks.append(bits_of(kf)), Vs.append(v.bits)
    Q, K, V = E.array(np.stack(Qs)), E.array(np.stack(Ks)), E.array(np.stack(Vs))
    O, L = E.empty((2, nq, h, d), np.uint16), E.empty((2, h, nq), np.float32)
    attention(E, Q, K, V, O, mode=AR, n_ar=n_ar, lse=L)
    for b, (qf, kf, vf) in enumerate(ins):
        want, lse = oattn.attention(qf, kf, vf, 0, AR, n_ar=n_ar)
        assert_parity(val(O[b]), want, "bf16", "large scores %s item %d" % (kind, b))
        np.testing.assert_allclose(L[b], lse, atol=BF16_LSE_ATOL, rtol=0)


def test_attention_bf16_edge_properties(E):
    """AR rows do not depend on DM rows (bitwise); the first row equals the
    first value row exactly; two runs give the same bits."""
    E.config(True, False)
    n, n_ar, h, d = 300, 100, 2, 128
    q, k, v = _qkv(9, n, n, h, h, d, "bf16")
    Q, K, V = E.array(q.bits), E.array(k.bits), E.array(v.bits)
    O1, O2, O3 = (E.empty((n, h, d), np.uint16) for _ in range(3))
    attention(E, Q, K, V, O1, mode=AR, n_ar=n_ar)
    attention(E, Q, K, V, O3, mode=AR, n_ar=n_ar)
    np.testing.assert_array_equal(O1, O3)
    np.testing.assert_array_equal(val(O1[0]), v.f32[0])
    Q2, K2, V2 = E.array(q.bits), E.array(k.bits), E.array(v.bits)
    Q2[n_ar:] = bits_of(val(Q2[n_ar:]) * 2)
    K2[n_ar:] = bits_of(-val(K2[n_ar:]))
    V2[n_ar:] = bits_of(val(V2[n_ar:]) + 3)
    attention(E, Q2, K2, V2, O2, mode=AR, n_ar=n_ar)
    np.testing.assert_array_equal(O1[:n_ar], O2[:n_ar])
    assert not np.array_equal(O1[n_ar:], O2[n_ar:])


F32_CASES = [
    ("f32_ar_d128", 150, 150, 0, AR, 40, 0, 0, 128, 3, 3),
    ("f32_ar_qoffset_d128", 70, 230, 160, AR, 100, 0, 0, 128, 3, 3),
    ("f32_chunk_d64", 3 * 37 + 5, 20 + 3 * 37 + 5, 20, CH, 0, 20, 37, 64, 3, 3),
    ("f32_chunk_d128", 2 * 45 + 7, 33 + 2 * 45 + 7, 33, CH, 0, 33, 45, 128, 2, 2),
    ("f32_gqa_d64", 90, 90, 0, AR, 30, 0, 0, 64, 6, 2),
    ("f32_ar_d80", 110, 110, 0, AR, 40, 0, 0, 80, 4, 2),
]


@pytest.mark.parametrize("case", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_attention_fp32(E, case):
    name, nq, nk, q0, mask, n_ar, n_prefix, cl, d, h, hk = case
    E.config(False, True)
    q, k, v = _qkv(12, nq, nk, h, hk, d, "fp32")
    Q, K, V = E.array(q.f32), E.array(k.f32), E.array(v.f32)
    O, L = E.empty((nq, h, d), np.float32), E.empty((h, nq), np.float32)
    attention(E, Q, K, V, O, mode=mask, q0=q0, n_ar=n_ar, n_prefix=n_prefix, chunk_len=cl, lse=L)
    want, lse = oattn.attention(q.f32, k.f32, v.f32, q0, mask, n_ar, n_prefix, max(cl, 1))
    assert_parity(O, want, "fp32", name)
    np.testing.assert_allclose(L, lse, atol=1e-4, rtol=0)


@pytest.mark.parametrize("d", [64, 80])
def test_attention_fp32_batched_rope_both(E, d):
    """fp32 with two batch items, GQA and mRoPE on load for Q and K."""
    E.config(False, False)
    n, h, hk = 120, 4, 2
    pos = np.ascontiguousarray(olayout.build(W.BY_NAME["policy_bf16"].segments)[0][:n])
    secs = (d // 8, 3 * d // 16, 3 * d // 16)
    ins = [_qkv(40 + b, n, n, h, hk, d, "fp32") for b in range(2)]
    Q = E.array(np.stack([t[0].f32 for t in ins]))
    K = E.array(np.stack([t[1].f32 for t in ins]))
    V = E.array(np.stack([t[2].f32 for t in ins]))
    P = E.array(pos)
    O = E.empty((2, n, h, d), np.float32)
    attention(E, Q, K, V, O, mode=AR, n_ar=40, q_pos=P, k_pos=P, sections=secs, theta=1e4)
    for b, (q, k, v) in enumerate(ins):
        want, _ = oattn.attention(omrope.apply(q.f32, pos, secs, 1e4), omrope.apply(k.f32, pos, secs, 1e4),
                                  v.f32, 0, AR, n_ar=40)
        assert_parity(O[b], want, "fp32", "fp32 batch %d" % b)


# ---------------------------------------------------------------------------
# merge
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("parts,d", [(2, 64), (3, 64), (16, 64), (3, 80)])
def test_merge(E, dt, parts, d):
    """Merge of per-part outputs through their LSE, with some parts holding
    no key for some rows (LSE -inf, NaN outputs that must not be read)."""
    E.config(False, False)
    nq, h = 37, 3
    r = np.random.default_rng(parts)
    o = W.make(50 + parts, 1, (parts, nq, h, d), dt)
    lse = (r.standard_normal((parts, h, nq)) * 3).astype(np.float32)
    lse[0, :, ::5] = -np.inf
    if parts > 2:
        lse[1:, 1, 3] = -np.inf
    of = (o.bits if dt == "bf16" else o.f32).copy()
    nan = np.uint16(0x7FC0) if dt == "bf16" else np.float32(np.nan)
    of[0][np.transpose(np.isneginf(lse[0]))] = nan
    Op, Lp = E.array(of), E.array(lse)
    O = E.empty((nq, h, d), of.dtype)
    L = E.empty((h, nq), np.float32)
    el = _el(Op)
    st = E.call("mot_attention_merge", emu_lib.ptr(Op), emu_lib.ptr(Lp), parts, el[0], nq, h, d, el[1], el[2],
                emu_lib.ptr(O), h * d, d, emu_lib.ptr(L), BF16 if dt == "bf16" else FP32, None)
    assert st == 0
    want, wl = oattn.merge(o.f32, lse)
    got = val(O) if dt == "bf16" else O
    assert_parity(got, want, dt, "merge")
    np.testing.assert_allclose(L, wl, atol=1e-5, rtol=1e-6)


# ---------------------------------------------------------------------------
# region-split projection
GEMM_CASES = [
    # n_rows, n_ar, K, N
    (300, 130, 256, 384),
    (260, 70, 64, 192),
    (129, 0, 128, 128),
    (200, 200, 192, 64),
    (1, 1, 64, 64),
    (511, 255, 128, 320),
]


def _gemm_inputs(case, dt, seed=3):
    n, n_ar, K, N = case
    x = W.make(seed, 1, (n, K), dt)
    wa = W.make(seed, 2, (K, N), dt, 1.0 / math.sqrt(K))
    wd = W.make(seed, 3, (K, N), dt, 1.0 / math.sqrt(K))
    return x, wa, wd


def region_linear(E, x, wa, wd, y, n_ar, in_dt, out_dt, epi=0, res=None):
    n, K = x.shape
    st = E.call("mot_region_linear", emu_lib.ptr(x), emu_lib.ptr(wa), emu_lib.ptr(wd), emu_lib.ptr(y), n, n_ar,
                K, y.shape[1], in_dt, out_dt, epi, emu_lib.ptr(res), None)
    assert st == 0, st


def _check_gemm(E, case, out_dt, epi, in_place):
    n, n_ar, K, N = case
    x, wa, wd = _gemm_inputs(case, "bf16")
    X, WA, WD = E.array(x.bits), E.array(wa.bits), E.array(wd.bits)
    want = oproj.project(x.f32, wa.f32, wd.f32, n_ar)
    res = None
    if epi == 1:
        want = oblock.gelu(want)
    elif epi == 2:
        rv = W.make(4, 5, (n, N), "bf16" if out_dt == BF16 else "fp32", 4.0)
        res = rv.bits if out_dt == BF16 else rv.f32
        want = want + rv.f32
    Y = E.empty((n, N), np.uint16 if out_dt == BF16 else np.float32)
    R = None
    if res is not None:
        if in_place:
            Y[...] = res
            R = Y
        else:
            R = E.array(res)
    region_linear(E, X, WA, WD, Y, n_ar, BF16, out_dt, epi, R)
    got = val(Y) if out_dt == BF16 else Y
    if out_dt == BF16 and epi == 2:
        assert_parity_stored(got, want, "gemm")
    else:
        assert_parity(got, want, "bf16", "gemm")
    if out_dt == BF16 and epi == 0:
        # the store is the round-to-nearest-even of the fp32 accumulator:
        # within one bf16 spacing of the exact value
        assert (np.abs(got - want) <= np.maximum(1e-6, 2.0 ** (np.floor(np.log2(np.abs(want) + 1e-30)) - 7))).all()


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "n%d_ar%d_K%d_N%d" % c)
def test_region_linear_bf16(E, case, mode):
    E.config(*mode)
    _check_gemm(E, case, BF16, 0, False)


@pytest.mark.parametrize("out_dt", [BF16, FP32], ids=["out_bf16", "out_fp32"])
@pytest.mark.parametrize("epi,in_place", [(1, False), (2, False), (2, True)], ids=["gelu", "add", "add_in_place"])
def test_region_linear_bf16_epilogues(E, out_dt, epi, in_place):
    E.config(True, True)
    _check_gemm(E, (300, 130, 128, 192), out_dt, epi, in_place)


@pytest.mark.parametrize("epi", [0, 1, 2])
@pytest.mark.parametrize("case", [(70, 30, 40, 50), (33, 0, 16, 17), (16, 16, 64, 32), (20, 20, 24, 8),
                                  (20, 0, 24, 8), (37, 19, 16, 16)],
                         ids=lambda c: "n%d_ar%d_K%d_N%d" % c)
def test_region_linear_fp32(E, case, epi):
    E.config(False, True)
    n, n_ar, K, N = case
    x, wa, wd = _gemm_inputs(case, "fp32")
    want = oproj.project(x.f32, wa.f32, wd.f32, n_ar)
    R = None
    if epi == 1:
        want = oblock.gelu(want)
    elif epi == 2:
        rv = W.make(4, 6, (n, N), "fp32")
        R = E.array(rv.f32)
        want = want + rv.f32
    Y = E.empty((n, N), np.float32)
    # a room with no rows passes NULL weights
    WA = E.array(wa.f32) if n_ar > 0 else None
    WD = E.array(wd.f32) if n_ar < n else None
    region_linear(E, E.array(x.f32), WA, WD, Y, n_ar, FP32, FP32, epi, R)
    assert_parity(Y, want, "fp32", "gemm fp32")


# The direct-to-LDS MFMA GEMM (built only with -DMOT_GEMM_DMA=1, switched off
# in the library until it has run on a GPU): the same checks on that build.
@pytest.fixture(scope="module")
def E_dma(tmp_path_factory):
    e = emu_lib.Emu(emu_lib.build(str(tmp_path_factory.mktemp("emu_dma")), dma_gemm=True))
    yield e
    e.free_all()


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("case", GEMM_CASES + [(600, 300, 256, 512)], ids=lambda c: "n%d_ar%d_K%d_N%d" % c)
def test_region_linear_dma_gemm_build(E_dma, case, mode):
    E_dma.config(*mode)
    try:
        before = E_dma.stat(emu_lib.ST_DMA)
        _check_gemm(E_dma, case, BF16, 0, False)
        assert E_dma.stat(emu_lib.ST_DMA) > before  # the direct-to-LDS kernel ran
    finally:
        E_dma.free_all()


@pytest.mark.parametrize("out_dt", [BF16, FP32], ids=["out_bf16", "out_fp32"])
@pytest.mark.parametrize("epi,in_place", [(1, False), (2, False), (2, True)], ids=["gelu", "add", "add_in_place"])
def test_region_linear_dma_gemm_build_epilogues(E_dma, out_dt, epi, in_place):
    E_dma.config(True, True)
    try:
        _check_gemm(E_dma, (300, 130, 128, 192), out_dt, epi, in_place)
    finally:
        E_dma.free_all()


# ---------------------------------------------------------------------------
# LayerNorm
@pytest.mark.parametrize("hidden", [64, 520, 1024, 4104, 8192])
@pytest.mark.parametrize("dts", [("bf16", BF16), ("fp32", FP32), ("bf16", FP32)], ids=["bf16", "fp32", "bf16_to_fp32"])
def test_layernorm_region(E, hidden, dts):
    E.config(False, False)
    in_name, out_dt = dts
    n, n_ar = 13, 5
    x = W.make(60, 1, (n, hidden), in_name, 3.0)
    r = np.random.default_rng(hidden)
    ga, ba, gd, bd = ((1 + 0.1 * r.standard_normal(hidden)).astype(np.float32),
                      (0.1 * r.standard_normal(hidden)).astype(np.float32),
                      (1 + 0.1 * r.standard_normal(hidden)).astype(np.float32),
                      (0.1 * r.standard_normal(hidden)).astype(np.float32))
    X = E.array(x.bits if in_name == "bf16" else x.f32)
    Y = E.empty((n, hidden), np.uint16 if out_dt == BF16 else np.float32)
    GA, BA, GD, BD = (E.array(t) for t in (ga, ba, gd, bd))
    st = E.call("mot_layernorm_region", emu_lib.ptr(X), emu_lib.ptr(Y), n, n_ar, hidden, emu_lib.ptr(GA),
                emu_lib.ptr(BA), emu_lib.ptr(GD), emu_lib.ptr(BD), ctypes.c_float(1e-6),
                BF16 if in_name == "bf16" else FP32, out_dt, None)
    assert st == 0
    want = oblock.region_layer_norm(x.f32, (ga, ba), (gd, bd), n_ar, 1e-6)
    got = val(Y) if out_dt == BF16 else Y
    assert_parity(got, want, "bf16" if out_dt == BF16 else "fp32", "layernorm")


# ---------------------------------------------------------------------------
# Euler updates
@pytest.mark.parametrize("n", [1, 7, 8, 4099])
@pytest.mark.parametrize("vdt", ["bf16", "fp32"])
@pytest.mark.parametrize("guided", [False, True])
def test_euler(E, n, vdt, guided):
    E.config(False, False)
    x0 = W.make(10, 1, (n,), "fp32").f32
    vc = W.make(10, 2, (n,), vdt)
    vb = W.make(10, 3, (n,), vdt)
    X = E.array(x0)
    XB = E.empty((n,), np.uint16)
    VC = E.array(vc.bits if vdt == "bf16" else vc.f32)
    VB = E.array(vb.bits if vdt == "bf16" else vb.f32)
    code = BF16 if vdt == "bf16" else FP32
    if guided:
        st = E.call("flow_cfg_euler_step", emu_lib.ptr(X), emu_lib.ptr(VC), emu_lib.ptr(VB), code, n,
                    ctypes.c_float(6.0), ctypes.c_float(0.9), ctypes.c_float(0.7), emu_lib.ptr(XB), None)
        want = ocfg.euler_step(x0, vc.f32, vb.f32, 6.0, 0.9, 0.7)
    else:
        st = E.call("flow_euler_step", emu_lib.ptr(X), emu_lib.ptr(VC), code, n, ctypes.c_float(1.0),
                    ctypes.c_float(0.75), emu_lib.ptr(XB), None)
        want = oeuler.step(x0, vc.f32, 1.0, 0.75)
    assert st == 0
    assert_parity(X, want, "fp32", "euler")
    np.testing.assert_array_equal(XB, W.bf16_bits(np.array(X)))  # the mirror is RNE of the new x


def test_euler_guidance_one_and_zero_velocity(E):
    """w = 0 takes v_base exactly (v = fma(w, v_cond - v_base, v_base); at
    w = 1 the rounded difference makes v_cond exact only up to one
    rounding); zero velocities leave x bitwise."""
    E.config(False, False)
    n = 1003
    x0 = W.make(14, 1, (n,), "fp32").f32
    vc = W.make(14, 2, (n,), "fp32").f32
    vb = W.make(14, 3, (n,), "fp32").f32
    X1, X2 = E.array(x0), E.array(x0)
    VC, VB = E.array(vc), E.array(vb)
    assert E.call("flow_cfg_euler_step", emu_lib.ptr(X1), emu_lib.ptr(VC), emu_lib.ptr(VB), FP32, n,
                  ctypes.c_float(0.0), ctypes.c_float(0.5), ctypes.c_float(0.25), None, None) == 0
    assert E.call("flow_euler_step", emu_lib.ptr(X2), emu_lib.ptr(VB), FP32, n, ctypes.c_float(0.5),
                  ctypes.c_float(0.25), None, None) == 0
    np.testing.assert_array_equal(X1, X2)
    X3, Z = E.array(x0), E.empty((n,), np.uint16)
    assert E.call("flow_euler_step", emu_lib.ptr(X3), emu_lib.ptr(Z), BF16, n, ctypes.c_float(0.5),
                  ctypes.c_float(0.25), None, None) == 0
    np.testing.assert_array_equal(X3.view(np.uint32), x0.view(np.uint32))


# ---------------------------------------------------------------------------
# mRoPE
@pytest.mark.parametrize("name", ["tiny_fp32", "policy_bf16", "super_t2v480p_bf16"])
def test_mrope_strided_views(E, name):
    E.config(False, False)
    wl = W.BY_NAME[name]
    pos, reg, n_ar = olayout.build(wl.segments)
    n = min(len(reg), 700)
    pos = np.ascontiguousarray(pos[:n])
    h, d = wl.n_heads, wl.head_dim
    y = W.make(wl.wid, 40, (n, 3, h, d), wl.dtype)
    Y = E.array(y.bits if wl.dtype == "bf16" else y.f32)
    P = E.array(pos)
    code = BF16 if wl.dtype == "bf16" else FP32
    for part in (0, 1):
        view = Y[:, part]
        el = _el(view)
        st = E.call("mrope_apply", emu_lib.ptr(view), code, n, h, d, el[0], el[1], emu_lib.ptr(P),
                    wl.sections[0], wl.sections[1], wl.sections[2], ctypes.c_float(wl.theta), None)
        assert st == 0
    got = val(Y) if wl.dtype == "bf16" else Y
    for part in (0, 1):
        want = omrope.apply(y.f32[:, part], pos, wl.sections, wl.theta)
        assert_parity(got[:, part], want, wl.dtype, "mrope part %d" % part)
    np.testing.assert_array_equal(got[:, 2], y.f32[:, 2])


# ---------------------------------------------------------------------------
# the whole MoT layer through the C ABI, as the layer step chains it
def test_whole_layer_chain_through_the_c_abi(E):
    """LayerNorm -> QKV projection -> mRoPE on K -> attention (mRoPE on Q on
    load) -> output projection + residual -> LayerNorm -> MLP up + GELU ->
    MLP down + residual, every intermediate stored in bf16, against the
    oracle's layer with bf16 storage at the same points."""
    E.config(True, True)
    h, d, hid, ffn = 2, 64, 128, 192
    secs, theta = (8, 12, 12), 1e4
    wl = W.BY_NAME["policy_bf16"]
    pos_all, reg, n_ar_all = olayout.build(wl.segments)
    n_ar, n = 70, 200
    pos = np.ascontiguousarray(np.concatenate([pos_all[:n_ar], pos_all[n_ar_all:n_ar_all + n - n_ar]]))
    r = np.random.default_rng(5)
    p = {}
    for room in ("ar", "dm"):
        p["ln1_" + room] = ((1 + 0.1 * r.standard_normal(hid)).astype(np.float32),
                            (0.1 * r.standard_normal(hid)).astype(np.float32))
        p["ln2_" + room] = ((1 + 0.1 * r.standard_normal(hid)).astype(np.float32),
                            (0.1 * r.standard_normal(hid)).astype(np.float32))
        for key, shape in (("qkv_", (hid, 3 * h * d)), ("o_", (h * d, hid)), ("up_", (hid, ffn)),
                           ("down_", (ffn, hid))):
            p[key + room] = val(bits_of(r.standard_normal(shape) / math.sqrt(shape[0])))
    X = val(bits_of(r.standard_normal((n, hid))))
    want = oblock.layer(X, p, pos, n_ar, h, d, secs, theta, store="bf16")

    dev = {k: (E.array(bits_of(v)) if not k.startswith("ln") else tuple(E.array(t) for t in v)) for k, v in p.items()}
    Xd = E.array(bits_of(X))
    P = E.array(pos)
    U1 = E.empty((n, hid), np.uint16)

    def ln(x, y, key):
        a, b = dev[key + "_ar"], dev[key + "_dm"]
        assert E.call("mot_layernorm_region", emu_lib.ptr(x), emu_lib.ptr(y), n, n_ar, hid, emu_lib.ptr(a[0]),
                      emu_lib.ptr(a[1]), emu_lib.ptr(b[0]), emu_lib.ptr(b[1]), ctypes.c_float(1e-6), BF16, BF16,
                      None) == 0

    ln(Xd, U1, "ln1")
    Y = E.empty((n, 3, h, d), np.uint16)
    region_linear(E, U1, dev["qkv_ar"], dev["qkv_dm"], Y.reshape(n, 3 * h * d), n_ar, BF16, BF16)
    K = Y[:, 1]
    el = _el(K)
    assert E.call("mrope_apply", emu_lib.ptr(K), BF16, n, h, d, el[0], el[1], emu_lib.ptr(P), *secs,
                  ctypes.c_float(theta), None) == 0
    O = E.empty((n, h, d), np.uint16)
    attention(E, Y[:, 0], K, Y[:, 2], O, mode=AR, n_ar=n_ar, q_pos=P, sections=secs, theta=theta)
    H1 = E.array(bits_of(X))
    region_linear(E, O.reshape(n, h * d), dev["o_ar"], dev["o_dm"], H1, n_ar, BF16, BF16, 2, H1)
    U2 = E.empty((n, hid), np.uint16)
    ln(H1, U2, "ln2")
    A = E.empty((n, ffn), np.uint16)
    region_linear(E, U2, dev["up_ar"], dev["up_dm"], A, n_ar, BF16, BF16, 1)
    H2 = E.array(np.array(H1))
    region_linear(E, A, dev["down_ar"], dev["down_dm"], H2, n_ar, BF16, BF16, 2, H2)

    assert_parity(val(U1), want["u1"], "bf16", "u1")
    assert_parity_stored(val(H1), want["h1"], "h1")
    # H2 = round(H1 + delta) on both sides, each H1 already within a spacing
    assert_parity_stored(val(H2), want["h2"], "h2", spacings=2)
    ma, rl = errors(val(H2) - X, want["h2"] - X)
    assert rl < 2e-2, rl  # the layer's update itself, not just the residual stream


# ---------------------------------------------------------------------------
# the emulator sees planted mistakes
PLANTED = [
    ("ragged tile not clamped", [("attn_tiles.hpp", "const int64_t rr = r > last ? last : r;",
                                  "const int64_t rr = r;")], "fault"),
    ("no vmcnt wait before the barrier", [("attention.hip", "    if (j < ntiles) {\n      wait_vmem0();\n",
                                           "    if (j < ntiles) {\n")], "wrong"),
    ("no barrier after the prologue", [("attention.hip",
                                        "  __syncthreads();  // every wave has read K(0) before step 0 overwrites "
                                        "its slot", "")], "wrong"),
    ("wrong key/value head", [("attention.hip", "head / p.kv_group)", "head % (p.n_heads / p.kv_group))")],
     "wrong"),
    ("K copy and read swizzles differ", [("attn_tiles.hpp", "(IS_K ? swz_k<DS>(r) : swz_v<DS>(r))",
                                          "(IS_K ? 0 : swz_v<DS>(r))")], "wrong"),
    ("D = 80 padding dims stored", [("attention.hip", "if (D % 32 != 0 && d0 >= D) continue;", "")], "wrong80"),
    ("D = 80 rotation partner on the wrong side", [("attention.hip", "(d < D / 2 ? d + D / 2 : d - D / 2)",
                                                    "(d < D / 2 ? d + D / 2 : d)")], "rope80"),
    ("GEMM epilogue residual row", [("gemm.hip", "store4<OUT_BF16, EPI>(p, row * p.N + n, o);\n      }\n  }\n}\n\n//",
                                     "store4<OUT_BF16, EPI>(p, (row ^ 1) * p.N + n, o);\n      }\n  }\n}\n\n//")],
     "gemm"),
    ("fp32 GEMM reads the absent room's weights past the last row",
     [("gemm.hip", "const int64_t rhi = rlo + FT < M ? rlo + FT : M;", "const int64_t rhi = rlo + FT;")],
     "gemm_f32_null"),
]


@pytest.mark.parametrize("what,patches,kind", PLANTED, ids=[p[0] for p in PLANTED])
def test_planted_mistake_is_caught(tmp_path, what, patches, kind):
    Ep = emu_lib.Emu(emu_lib.build(str(tmp_path / "b"), patches=patches))
    try:
        caught = []
        for mode in MODES:
            Ep.config(*mode)
            try:
                if kind == "gemm":
                    _check_gemm(Ep, (300, 130, 128, 192), BF16, 0, False)
                elif kind == "gemm_f32_null":
                    x, wa, _ = _gemm_inputs((20, 20, 24, 8), "fp32")
                    Y = Ep.empty((20, 8), np.float32)
                    region_linear(Ep, Ep.array(x.f32), Ep.array(wa.f32), None, Y, 20, FP32, FP32)
                    assert_parity(Y, oproj.project(x.f32, wa.f32, wa.f32, 20), "fp32", what)
                elif kind == "rope80":
                    n, h, d = 200, 2, 80
                    pos = np.ascontiguousarray(olayout.build(W.BY_NAME["policy_bf16"].segments)[0][:n])
                    secs = (10, 15, 15)
                    q, k, v = _qkv(8, n, n, h, h, d, "bf16")
                    kb = bits_of(omrope.apply(k.f32, pos, secs, 1e4))
                    O = Ep.empty((n, h, d), np.uint16)
                    attention(Ep, Ep.array(q.bits), Ep.array(kb), Ep.array(v.bits), O, mode=AR, n_ar=60,
                              q_pos=Ep.array(pos), sections=secs, theta=1e4)
                    want, _ = oattn.attention(omrope.apply(q.f32, pos, secs, 1e4), val(kb), v.f32, 0, AR, 60)
                    assert_parity(val(O), want, "bf16", what)
                else:
                    nq, h, hk, d = 300, 8, 2, 80 if kind == "wrong80" else 128
                    q, k, v = _qkv(7, nq, nq, h, hk, d, "bf16")
                    Q, K, V = Ep.array(q.bits), Ep.array(k.bits), Ep.array(v.bits)
                    O = Ep.empty((nq, h, d), np.uint16)
                    attention(Ep, Q, K, V, O, mode=AR, n_ar=70)
                    want, _ = oattn.attention(q.f32, k.f32, v.f32, 0, AR, 70)
                    assert_parity(val(O), want, "bf16", what)
                caught.append(False)
            except AssertionError as e:
                caught.append(("memory fault" in str(e)) if kind == "fault" else True)
            Ep.free_all()
        assert any(caught), what
    finally:
        Ep.free_all()


# ---------------------------------------------------------------------------
def test_results_do_not_depend_on_scheduling(E):
    """Every kernel's output is the same bits whatever the wave order between
    barriers and whenever the LDS-DMA copies land (no result depends on
    timing: no atomics, no order-dependent reductions across waves)."""
    modes = [(False, False), (True, True), (True, 2), (False, 2)]
    nq, h, hk, d = 260, 8, 2, 128
    q, k, v = _qkv(70, nq, nq, h, hk, d, "bf16")
    x, wa, wd = _gemm_inputs((300, 130, 128, 192), "bf16", seed=71)
    outs = []
    for mode in modes:
        E.config(*mode)
        Q, K, V = E.array(q.bits), E.array(k.bits), E.array(v.bits)
        O, L = E.empty((nq, h, d), np.uint16), E.empty((h, nq), np.float32)
        attention(E, Q, K, V, O, mode=AR, n_ar=90, lse=L)
        O2 = E.empty((nq, h, d), np.uint16)
        attention(E, Q, K, V, O2, mode=CH, q0=40, n_prefix=40, chunk_len=50)
        Y = E.empty((300, 192), np.uint16)
        region_linear(E, E.array(x.bits), E.array(wa.bits), E.array(wd.bits), Y, 130, BF16, BF16, 1)
        outs.append([np.array(t) for t in (O, L, O2, Y)])
        E.free_all()
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            np.testing.assert_array_equal(a.view(np.uint8), b.view(np.uint8))
