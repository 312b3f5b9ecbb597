"""Full-size attention launches on sampled workgroups, on the CPU emulator.

The launch runs at its real grid and shapes, but the emulator executes only
a strided sample of its workgroups (tests/native/emu, emu_subset). The
others are skipped, and the output rows they would write keep their NaN
fill. Every (row, head) the sample writes is compared with the oracle.
Launches:

* the 480p text-to-video step's attention: 25,474 tokens, 24 heads of 128,
  Q, K, V strided views of the packed projection output, Q rotated on load;
* the same layout at the Super head shape (64 / 8 heads of 80);
* the streaming chunk against the full rolling cache (1,440 queries,
  13,218 keys, chunk-causal mask);
* (MOT_EMU_FULLSIZE=1) the long 480p sequence, 76,954 tokens.

The grid is ordered heaviest first: query tile qt = n_qtiles - 1 - x / H,
so the small x are the last (ragged) DM tiles and the large x the AR tiles.
Each launch runs one sample from each end and one strided across the
middle, so the sample takes the ragged last tile, full DM tiles, the tile
holding the AR/DM boundary, and causal AR tiles.
"""
import os

import numpy as np
import pytest

import workloads as W
from oracle import attention as oattn
from oracle import layout as olayout
from oracle import mrope as omrope
from tests import emu_lib
from tests.gpu_util import assert_parity

pytestmark = pytest.mark.skipif(not os.path.exists(emu_lib.CXX), reason="host clang++ missing")
pytest.importorskip("multimodal_diffusion_transformer_amd._binding")

AR, CH = W.AR_CAUSAL_DM_FULL, W.CHUNK_CAUSAL_KV
BM = 128  # query rows per workgroup


@pytest.fixture(scope="module")
def E(tmp_path_factory):
    e = emu_lib.Emu(emu_lib.build(str(tmp_path_factory.mktemp("emu_full"))))
    e.config(True, True)  # copies held until their wait, waves in reverse
    yield e
    e.subset(0)
    e.free_all()


def _launch_sampled(E, samples, **kw):
    """One launch per (stride, offset, count) sample, into the same output."""
    from tests.test_emu_kernels import attention
    for stride, offset, count in samples:
        E.subset(stride, offset, count)
        try:
            attention(E, **kw)
        finally:
            E.subset(0)


def _written(O):
    """(rows, heads) with every output dim written (not NaN), grouped per
    head; each head's rows must be whole 128-row tiles (the last may be
    ragged)."""
    vals = W.bf16_to_f32(np.asarray(O))
    done = ~np.isnan(vals).any(axis=-1)            # [nq, H]
    assert not (np.isnan(vals).any(axis=-1) & ~np.isnan(vals).all(axis=-1)).any(), "partly written rows"
    nq = O.shape[0]
    per_head = {}
    for h in range(O.shape[1]):
        rows = np.nonzero(done[:, h])[0]
        if len(rows) == 0:
            continue
        tiles = np.unique(rows // BM)
        for t in tiles:
            want = np.arange(t * BM, min(nq, (t + 1) * BM))
            assert np.array_equal(rows[(rows >= t * BM) & (rows < (t + 1) * BM)], want), (h, t)
        per_head[h] = rows
    return vals, per_head


def _samples(n_qtiles, h, mid=6):
    x_total = n_qtiles * h
    return [(1, 0, 2),                                            # the last (ragged) DM tile
            (x_total // mid + 1, h + 3, mid),                     # strided across the middle
            (h + 1, x_total - 5 * h, 5)]                          # query tiles 4..0: AR rows and the boundary


def _packed_case(E, wl, seed):
    """The step's launch at workload wl: Q, K, V strided views of one packed
    [N, (H + 2 H_kv) D] buffer, Q rotated on load, K as given."""
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h, hk, d = len(reg), wl.n_heads, wl.kv_heads, wl.head_dim
    q = W.make(seed, W.T_Q, (n, h, d), "bf16")
    k = W.make(seed, W.T_K, (n, hk, d), "bf16")
    v = W.make(seed, W.T_V, (n, hk, d), "bf16")
    Y = E.empty((n, (h + 2 * hk) * d), np.uint16)
    Y[:, :h * d] = q.bits.reshape(n, h * d)
    Y[:, h * d:(h + hk) * d] = k.bits.reshape(n, hk * d)
    Y[:, (h + hk) * d:] = v.bits.reshape(n, hk * d)
    O = E.array(np.full((n, h, d), 0xFFFF, np.uint16))   # NaN
    P = E.array(np.ascontiguousarray(pos))
    qv = Y[:, :h * d].reshape(n, h, d)
    kv_ = Y[:, h * d:(h + hk) * d].reshape(n, hk, d)
    vv = Y[:, (h + hk) * d:].reshape(n, hk, d)
    n_qtiles = (n + BM - 1) // BM
    g0 = E.stat(1)  # workgroups run so far
    _launch_sampled(E, _samples(n_qtiles, h), q=qv, k=kv_, v=vv, o=O, mode=AR, n_ar=n_ar, q_pos=P,
                    sections=wl.sections, theta=wl.theta)
    ran = E.stat(1) - g0
    vals, per_head = _written(O)
    assert len(per_head) >= 4
    checked = 0
    for head, rows in sorted(per_head.items()):
        kvh = head // (h // hk)
        qr = omrope.apply(q.f32[rows][:, [head]], pos[rows], wl.sections, wl.theta)
        want = oattn.attention_rows(qr, k.f32[:, [kvh]], v.f32[:, [kvh]], rows, [0], 0, AR, n_ar=n_ar)
        assert_parity(vals[rows][:, [head]], want, "bf16", "%s head %d, %d rows" % (wl.name, head, len(rows)))
        checked += len(rows)
    tiles = {(hd, t) for hd, rows in per_head.items() for t in np.unique(rows // BM)}
    assert len(tiles) == ran == 2 + 6 + 5  # one (head, query tile) per workgroup run, none elsewhere
    qt_set = {t for _, t in tiles}
    # the ragged last tile, causal AR rows, the tile holding the AR/DM boundary
    assert {n_qtiles - 1, 0, n_ar // BM} <= qt_set, sorted(qt_set)
    return checked


@pytest.mark.parametrize("name", ["t2v480p_bf16", "super_t2v480p_bf16"])
def test_480p_step_attention_on_sampled_workgroups(E, name):
    checked = _packed_case(E, W.BY_NAME[name], 35)
    assert checked >= 8 * BM


@pytest.mark.skipif(os.environ.get("MOT_EMU_FULLSIZE") != "1", reason="long 480p: set MOT_EMU_FULLSIZE=1")
def test_long_480p_attention_on_sampled_workgroups(E):
    checked = _packed_case(E, W.BY_NAME["t2v480p_long_bf16"], 36)
    assert checked >= 8 * BM


def test_streaming_chunk_against_the_full_cache_on_sampled_workgroups(E):
    """The streaming call: the newest chunk (1,440 rows) against the rolling
    cache [prefix 258 | 8 history frames | chunk], chunk-causal mask, Q
    rotated on load at the chunk's positions."""
    wl = W.BY_NAME["stream_chunk_bf16"]
    pos, reg, n_ar = olayout.build(wl.segments)
    nk, h, d = len(reg), wl.n_heads, wl.head_dim
    ft = wl.stream_views * wl.stream_gh * wl.stream_gw
    n_prefix = wl.stream_text + 2
    q0 = nk - ft
    q = W.make(38, W.T_Q, (ft, h, d), "bf16")
    k = W.make(38, W.T_K, (nk, h, d), "bf16")
    v = W.make(38, W.T_V, (nk, h, d), "bf16")
    qpos = np.ascontiguousarray(pos[q0:])
    O = E.array(np.full((ft, h, d), 0xFFFF, np.uint16))
    n_qtiles = (ft + BM - 1) // BM
    _launch_sampled(E, [(n_qtiles * h // 5 + 1, 2, 5), (1, 0, 1), (1, n_qtiles * h - 1, 1)],
                    q=E.array(q.bits), k=E.array(k.bits), v=E.array(v.bits), o=O, mode=CH, q0=q0,
                    n_prefix=n_prefix, chunk_len=ft, q_pos=E.array(qpos), sections=wl.sections,
                    theta=wl.theta)
    vals, per_head = _written(O)
    assert len(per_head) >= 3
    for head, rows in sorted(per_head.items()):
        qr = omrope.apply(q.f32[rows][:, [head]], qpos[rows], wl.sections, wl.theta)
        want = oattn.attention_rows(qr, k.f32[:, [head]], v.f32[:, [head]], rows, [0], q0, CH,
                                    n_prefix=n_prefix, chunk_len=ft)
        assert_parity(vals[rows][:, [head]], want, "bf16", "stream head %d, %d rows" % (head, len(rows)))


BY_HAND = pytest.mark.skipif(os.environ.get("MOT_EMU_FULLSIZE") != "1", reason="set MOT_EMU_FULLSIZE=1")


@pytest.mark.parametrize("name", ["t2v480p_bf16", pytest.param("super_t2v480p_bf16", marks=BY_HAND),
                                  pytest.param("t2v480p_long_bf16", marks=BY_HAND)])
def test_480p_projections_on_sampled_workgroups(E, name):
    """The step's two region-split projections at full size, the first 514
    rows through the Reasoner's weights: at 480p QKV [25,474 x 3,072] x
    [3,072 x 9,216] and O [25,474 x 3,072] x [3,072 x 3,072]; the Super
    heads' [.. x 5,120] x [5,120 x 6,400] and x [5,120 x 5,120]; the long
    sequence's 76,954 rows.  Both rooms' tiles are in the sample (the grid
    lists the AR problem's tiles first); each written 128 x 128 output tile
    is compared with the oracle at the stored-bf16 bound."""
    from tests.gpu_util import assert_parity_stored
    from tests.test_emu_kernels import region_linear
    from oracle import projection as oproj
    wl = W.BY_NAME[name]
    n, hid, h, d, hk = wl.n_tokens, wl.hidden, wl.n_heads, wl.head_dim, wl.kv_heads
    n_ar = W.region_counts(wl.segments)[0]
    X = W.make(wl.wid, W.T_X, (n, hid), "bf16")
    for name, tid_ar, tid_dm, d_in, d_out in (("qkv", W.T_WQKV_AR, W.T_WQKV_DM, hid, (h + 2 * hk) * d),
                                              ("o", W.T_WO_AR, W.T_WO_DM, h * d, hid)):
        wa = W.make(wl.wid, tid_ar, (d_in, d_out), "bf16", 0.02)
        wd = W.make(wl.wid, tid_dm, (d_in, d_out), "bf16", 0.02)
        x = X if d_in == hid else W.make(wl.wid, W.T_Q, (n, d_in), "bf16")
        Y = E.array(np.full((n, d_out), 0xFFFF, np.uint16))
        tn = d_out // 128
        ar_tiles = (n_ar + 127) // 128 * tn
        total = ar_tiles + (n - n_ar + 127) // 128 * tn
        Xe, WA, WD = E.array(x.bits), E.array(wa.bits), E.array(wd.bits)
        for stride, offset, count in ((tn + 1, 0, (ar_tiles + tn) // (tn + 1)),   # the AR problem
                                      (total // 8 + 1, ar_tiles, 8),             # the DM problem
                                      (1, total - 2, 2)):                        # its last (ragged) row tile
            E.subset(stride, offset, count)
            try:
                region_linear(E, Xe, WA, WD, Y, n_ar, 0, 0)
            finally:
                E.subset(0)
        got = W.bf16_to_f32(np.asarray(Y))
        done = ~np.isnan(got)
        rows = np.nonzero(done.any(axis=1))[0]
        assert (rows < n_ar).any() and (rows >= n_ar).any() and rows[-1] == n - 1, name
        checked = 0
        # row tiles: 128-row tiles of each room (AR rows [0, n_ar), DM rows
        # from n_ar), the last of each possibly ragged
        tile_of = np.where(rows < n_ar, rows // 128, (n_ar + 127) // 128 + (rows - n_ar) // 128)
        for t in np.unique(tile_of):
            r0 = t * 128 if t < (n_ar + 127) // 128 else n_ar + (t - (n_ar + 127) // 128) * 128
            r1 = min(n_ar if r0 < n_ar else n, r0 + 128)
            rr = np.arange(r0, r1)
            for c0 in np.unique(np.nonzero(done[rr].any(axis=0))[0] // 128) * 128:
                blk = got[np.ix_(rr, np.arange(c0, c0 + 128))]
                assert not np.isnan(blk).any(), (name, r0, c0)   # whole tiles
                # a tile never straddles the room boundary: each row's room
                want = np.concatenate([oproj.project_rows(x.f32[rr[rr < n_ar]], wa.f32[:, c0:c0 + 128]),
                                       oproj.project_rows(x.f32[rr[rr >= n_ar]], wd.f32[:, c0:c0 + 128])])
                assert_parity_stored(blk, want, "%s tile (%d, %d)" % (name, r0, c0))
                checked += 1
        assert checked >= 10, (name, checked)


def test_480p_mrope_and_euler_whole_launches(E):
    """The step's two bandwidth kernels at 480p, every workgroup: mRoPE of K
    in the packed projection output (25,474 tokens x 24 heads, in place,
    strided view) and the Euler update of the 24,960 x 3,072 latent with its
    bf16 mirror."""
    from oracle import euler as oeuler
    import ctypes
    wl = W.BY_NAME["t2v480p_bf16"]
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h, d, hid = len(reg), wl.n_heads, wl.head_dim, wl.hidden
    k = W.make(40, W.T_K, (n, h, d), "bf16")
    Y = E.empty((n, 3, h, d), np.uint16)
    Y[:, 1] = k.bits
    P = E.array(np.ascontiguousarray(pos))
    view = Y[:, 1]
    st = E.call("mrope_apply", emu_lib.ptr(view), 0, n, h, d, 3 * h * d, d, emu_lib.ptr(P), *wl.sections,
                ctypes.c_float(wl.theta), None)
    assert st == 0
    assert_parity(W.bf16_to_f32(np.asarray(Y[:, 1])), omrope.apply(k.f32, pos, wl.sections, wl.theta), "bf16",
                  "mrope K 480p")
    assert (Y[:, 0] == 0).all() and (Y[:, 2] == 0).all()   # Q and V untouched
    n_noisy = W.region_counts(wl.segments)[2]
    x0 = W.make(wl.wid, W.T_LATENT, (n_noisy * hid,), "fp32").f32
    v = W.make(41, 1, (n_noisy * hid,), "bf16")
    X, V, XB = E.array(x0), E.array(v.bits), E.empty((n_noisy * hid,), np.uint16)
    st = E.call("flow_euler_step", emu_lib.ptr(X), emu_lib.ptr(V), 0, n_noisy * hid, ctypes.c_float(1.0),
                ctypes.c_float(0.975), emu_lib.ptr(XB), None)
    assert st == 0
    assert_parity(np.asarray(X), oeuler.step(x0, v.f32, 1.0, 0.975), "fp32", "euler 480p")
    np.testing.assert_array_equal(np.asarray(XB), W.bf16_bits(np.asarray(X)))


def _tiles_checked(got, want_fn, n, n_ar, d_out, what):
    """Compare every written 128 x 128 tile of a region GEMM output (rows
    tiled per room) with want_fn(rows, c0) at the stored-bf16 bound."""
    from tests.gpu_util import assert_parity_stored
    done = ~np.isnan(got)
    rows = np.nonzero(done.any(axis=1))[0]
    n_ar_t = (n_ar + 127) // 128
    tile_of = np.where(rows < n_ar, rows // 128, n_ar_t + (rows - n_ar) // 128)
    checked = 0
    for t in np.unique(tile_of):
        r0 = t * 128 if t < n_ar_t else n_ar + (t - n_ar_t) * 128
        rr = np.arange(r0, min(n_ar if r0 < n_ar else n, r0 + 128))
        for c0 in np.unique(np.nonzero(done[rr].any(axis=0))[0] // 128) * 128:
            blk = got[np.ix_(rr, np.arange(c0, min(d_out, c0 + 128)))]
            assert not np.isnan(blk).any(), (what, r0, c0)
            assert_parity_stored(blk, want_fn(rr, c0), "%s tile (%d, %d)" % (what, r0, c0))
            checked += 1
    return checked


@pytest.mark.skipif(os.environ.get("MOT_EMU_FULLSIZE") != "1", reason="whole-layer kernels: set MOT_EMU_FULLSIZE=1")
@pytest.mark.parametrize("name", ["nano_t2v480p_bf16", "super_t2v480p_bf16"])
def test_layer_kernels_at_480p(E, name):
    """The rest of the layer at the model table's shapes on the 480p layout
    (25,474 rows): LayerNorm of every row (whole launch), the MLP up
    projection with its GELU epilogue and the down projection with its
    residual epilogue on sampled tiles of both rooms, and the guided Euler
    update of the whole latent (whole launch)."""
    import ctypes
    from tests.test_emu_kernels import region_linear
    from oracle import block as oblock
    from oracle import cfg as ocfg
    from oracle import projection as oproj
    wl = W.BY_NAME[name]
    n, hid, ffn = wl.n_tokens, wl.hidden, wl.ffn
    n_ar, _, n_noisy = W.region_counts(wl.segments)
    p = W.block_params(wl)
    X = W.make(wl.wid, W.T_X, (n, hid), "bf16")
    # LayerNorm, every row
    U = E.empty((n, hid), np.uint16)
    (ga, ba), (gd, bd) = p["ln1_ar"], p["ln1_dm"]
    st = E.call("mot_layernorm_region", emu_lib.ptr(E.array(X.bits)), emu_lib.ptr(U), n, n_ar, hid,
                emu_lib.ptr(E.array(ga.f32)), emu_lib.ptr(E.array(ba.f32)), emu_lib.ptr(E.array(gd.f32)),
                emu_lib.ptr(E.array(bd.f32)), ctypes.c_float(1e-6), 0, 0, None)
    assert st == 0
    u = W.bf16_to_f32(np.asarray(U))
    want_u = oblock.region_layer_norm(X.f32, (ga.f32, ba.f32), (gd.f32, bd.f32), n_ar, 1e-6)
    assert_parity(u, want_u, "bf16", "%s ln1, every row" % name)

    def sampled(epi, x, wa, wd, d_out, res=None):
        Y = E.array(np.full((n, d_out), 0xFFFF, np.uint16))
        R = None if res is None else E.array(res)
        tn = d_out // 128
        ar_tiles = (n_ar + 127) // 128 * tn
        total = ar_tiles + (n - n_ar + 127) // 128 * tn
        Xe, WA, WD = E.array(x), E.array(wa), E.array(wd)
        for stride, offset, count in ((tn + 1, 0, 4), (total // 6 + 1, ar_tiles + 5, 6), (1, total - 1, 1)):
            E.subset(stride, offset, count)
            try:
                region_linear(E, Xe, WA, WD, Y, n_ar, 0, 0, epi, R)
            finally:
                E.subset(0)
        return Y

    up_a, up_d = p["up_ar"], p["up_dm"]
    A = sampled(1, U, up_a.bits, up_d.bits, ffn)
    a = W.bf16_to_f32(np.asarray(A))
    room = lambda rr, c0, wa_, wd_, x_: np.concatenate(
        [oproj.project_rows(x_[rr[rr < n_ar]], wa_[:, c0:c0 + 128]),
         oproj.project_rows(x_[rr[rr >= n_ar]], wd_[:, c0:c0 + 128])])
    k1 = _tiles_checked(a, lambda rr, c0: oblock.gelu(room(rr, c0, up_a.f32, up_d.f32, u)), n, n_ar, ffn,
                        "%s mlp up + gelu" % name)
    # the down projection over a full activation block, with the residual
    A_full = W.make(wl.wid, 60, (n, ffn), "bf16")
    H1 = W.make(wl.wid, 61, (n, hid), "bf16", 4.0)
    dn_a, dn_d = p["down_ar"], p["down_dm"]
    H2 = sampled(2, A_full.bits, dn_a.bits, dn_d.bits, hid, res=H1.bits)
    h2 = W.bf16_to_f32(np.asarray(H2))
    k2 = _tiles_checked(h2, lambda rr, c0: H1.f32[np.ix_(rr, np.arange(c0, c0 + 128))] +
                        room(rr, c0, dn_a.f32, dn_d.f32, A_full.f32), n, n_ar, hid, "%s mlp down + residual" % name)
    assert k1 >= 8 and k2 >= 8, (k1, k2)
    # guided Euler, the whole latent
    m = n_noisy * hid
    x0 = W.make(wl.wid, W.T_LATENT, (m,), "fp32").f32
    vc, vb = W.make(62, 1, (m,), "bf16"), W.make(62, 2, (m,), "bf16")
    Xl, XB = E.array(x0), E.empty((m,), np.uint16)
    st = E.call("flow_cfg_euler_step", emu_lib.ptr(Xl), emu_lib.ptr(E.array(vc.bits)), emu_lib.ptr(E.array(vb.bits)),
                0, m, ctypes.c_float(wl.guidance), ctypes.c_float(1.0), ctypes.c_float(0.975), emu_lib.ptr(XB), None)
    assert st == 0
    assert_parity(np.asarray(Xl), ocfg.euler_step(x0, vc.f32, vb.f32, wl.guidance, 1.0, 0.975), "fp32",
                  "%s guided euler" % name)
    np.testing.assert_array_equal(np.asarray(XB), W.bf16_bits(np.asarray(Xl)))


@pytest.mark.skipif(os.environ.get("MOT_EMU_FULLSIZE") != "1", reason="guided pair at 480p: set MOT_EMU_FULLSIZE=1")
@pytest.mark.parametrize("name", ["nano_t2v480p_bf16", "super_t2v480p_bf16"])
def test_guided_pair_attention_at_480p_on_sampled_workgroups(E, name):
    """Both predictions of a guided step in one launch at 480p: one packed
    buffer [AR cond | DM | AR base] of (N + n_ar) rows; item 0 reads keys
    [0, N), item 1 keys [n_ar, n_ar + N) (overlapping views, batch stride
    n_ar rows); the DM rows' Q shared (batch stride 0), rotated on load."""
    from tests.test_emu_kernels import attention
    wl = W.BY_NAME[name]
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h, hk, d = len(reg), wl.n_heads, wl.kv_heads, wl.head_dim
    n_dm = n - n_ar
    rows_all = n + n_ar
    width = (h + 2 * hk) * d
    q = W.make(39, W.T_Q, (n_dm, h, d), "bf16")
    k = W.make(39, W.T_K, (rows_all, hk, d), "bf16")
    v = W.make(39, W.T_V, (rows_all, hk, d), "bf16")
    Y = E.empty((rows_all, width), np.uint16)
    Y[n_ar:n_ar + n_dm, :h * d] = q.bits.reshape(n_dm, h * d)
    Y[:, h * d:(h + hk) * d] = k.bits.reshape(rows_all, hk * d)
    Y[:, (h + hk) * d:] = v.bits.reshape(rows_all, hk * d)
    st = np.lib.stride_tricks
    it = Y.itemsize
    qv = st.as_strided(Y[n_ar:], (2, n_dm, h, d), (0, width * it, d * it, it))
    kv_ = st.as_strided(Y[:, h * d:], (2, n, hk, d), (n_ar * width * it, width * it, d * it, it))
    vv = st.as_strided(Y[:, (h + hk) * d:], (2, n, hk, d), (n_ar * width * it, width * it, d * it, it))
    O = E.array(np.full((2, n_dm, h, d), 0xFFFF, np.uint16))
    P = E.array(np.ascontiguousarray(pos[n_ar:]))
    n_qtiles = (n_dm + BM - 1) // BM
    per_item = n_qtiles * h
    samples = [(per_item // 4 + 1, 1, 4), (1, per_item - 1, 1),                  # item 0
               (per_item // 4 + 1, per_item + 3, 4), (1, 2 * per_item - 2, 2)]   # item 1
    _launch_sampled(E, samples, q=qv, k=kv_, v=vv, o=O, mode=AR, q0=n_ar, n_ar=n_ar, q_pos=P,
                    sections=wl.sections, theta=wl.theta)
    checked = 0
    for b in range(2):
        vals, per_head = _written(O[b])
        assert per_head, b
        keys = slice(b * n_ar, b * n_ar + n)
        for head, rows in sorted(per_head.items()):
            kvh = head // (h // hk)
            qr = omrope.apply(q.f32[rows][:, [head]], pos[n_ar + rows], wl.sections, wl.theta)
            want = oattn.attention_rows(qr, k.f32[keys][:, [kvh]], v.f32[keys][:, [kvh]], n_ar + rows, [0], 0, AR,
                                        n_ar=n_ar)
            assert_parity(vals[rows][:, [head]], want, "bf16", "%s item %d head %d" % (name, b, head))
            checked += len(rows)
    assert checked >= 8 * BM


def test_streaming_chunk_key_split_and_merge_on_sampled_workgroups(E):
    """The streaming call with its keys split in two (the key-split path of
    the streaming cache): one launch of two items over the two halves of the
    13,218-key cache, Q shared, each half plain full attention (the chunk is
    the newest); the sample runs the same (query tile, head) workgroups of
    both items; then mot_attention_merge of all rows.  The merged rows of
    the sampled tiles are compared with attention over all keys."""
    wl = W.BY_NAME["stream_chunk_bf16"]
    pos, reg, _ = olayout.build(wl.segments)
    nk, h, d = len(reg), wl.n_heads, wl.head_dim
    ft = wl.stream_views * wl.stream_gh * wl.stream_gw
    n_prefix = wl.stream_text + 2
    q0 = nk - ft
    half = nk // 2
    q = W.make(42, W.T_Q, (ft, h, d), "bf16")
    k = W.make(42, W.T_K, (nk, h, d), "bf16")
    v = W.make(42, W.T_V, (nk, h, d), "bf16")
    qpos = np.ascontiguousarray(pos[q0:])
    Q, K, V = E.array(q.bits), E.array(k.bits), E.array(v.bits)
    st = np.lib.stride_tricks
    Qb = st.as_strided(Q, (2, ft, h, d), (0,) + Q.strides)
    Kb = st.as_strided(K, (2, half, h, d), (half * K.strides[0],) + K.strides)
    Vb = st.as_strided(V, (2, half, h, d), (half * V.strides[0],) + V.strides)
    Op = E.array(np.full((2, ft, h, d), 0xFFFF, np.uint16))
    Lp = E.array(np.full((2, h, ft), np.nan, np.float32))
    per_item = ((ft + BM - 1) // BM) * h
    # the same workgroup of both items: offsets x and x + per_item
    _launch_sampled(E, [(per_item, x, 2) for x in (0, 7, per_item // 2 + 5, per_item - 1)], q=Qb, k=Kb, v=Vb,
                    o=Op, mode=AR, q0=0, n_ar=0, q_pos=E.array(qpos), sections=wl.sections, theta=wl.theta,
                    lse=Lp)
    O = E.array(np.full((ft, h, d), 0xFFFF, np.uint16))
    L = E.array(np.full((h, ft), np.nan, np.float32))
    el = [s_ // Op.itemsize for s_ in Op.strides]
    st_ = E.call("mot_attention_merge", emu_lib.ptr(Op), emu_lib.ptr(Lp), 2, el[0], ft, h, d, el[1], el[2],
                 emu_lib.ptr(O), h * d, d, emu_lib.ptr(L), 0, None)
    assert st_ == 0
    _, parts = _written(Op[0])
    vals = W.bf16_to_f32(np.asarray(O))
    checked = 0
    for head, rows in sorted(parts.items()):
        assert not np.isnan(W.bf16_to_f32(np.asarray(Op[1]))[rows][:, head]).any()   # both halves ran
        qr = omrope.apply(q.f32[rows][:, [head]], qpos[rows], wl.sections, wl.theta)
        want = oattn.attention_rows(qr, k.f32[:, [head]], v.f32[:, [head]], rows, [0], q0, CH,
                                    n_prefix=n_prefix, chunk_len=ft)
        assert_parity(vals[rows][:, [head]], want, "bf16", "split + merge head %d" % head)
        checked += len(rows)
    assert checked >= 2 * BM
