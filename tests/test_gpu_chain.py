"""GPU parity of the chained one-layer denoiser step (projection -> mRoPE ->
attention -> output projection -> Euler) and of the streaming rollout,
teacher-forced step by step against the oracle.

End to end, a step's velocity is held to the bf16 contract (max-abs 2e-2,
relative L2 5e-3) against the oracle chain with bf16 activations
(``store="bf16"``: Y, the rotated Q and K, O and Z rounded where the bf16
path stores them).  What remains between the two is the bf16 rounding of the
softmax weights inside the attention kernel and the rounding flips it causes
downstream; a numpy model of the kernels' rounding points puts that at
rel-L2 3.2e-3 on the policy workload.  Against the unrounded fp64 chain the
same model gives 5.1e-3 (5.008e-3 was measured on the GPU), which is
reported, not asserted."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as oattn
from oracle import denoiser as oden
from oracle import euler as oeuler
from oracle import layout as olayout
from oracle import mrope as omrope
from oracle import projection as oproj
from oracle import streaming as ostream
from tests.gpu_util import assert_parity, device, errors, say, stream_workload, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _pipeline():
    from multimodal_diffusion_transformer_amd import pipeline
    return pipeline


def _inputs(wl):
    n = wl.n_tokens
    hid, h, d = wl.hidden, wl.n_heads, wl.head_dim
    X = W.make(wl.wid, W.T_X, (n, hid), wl.dtype)
    ws = [W.make(wl.wid, W.T_WQKV_AR, (hid, 3 * h * d), wl.dtype, 0.02),
          W.make(wl.wid, W.T_WQKV_DM, (hid, 3 * h * d), wl.dtype, 0.02),
          W.make(wl.wid, W.T_WO_AR, (h * d, hid), wl.dtype, 0.02),
          W.make(wl.wid, W.T_WO_DM, (h * d, hid), wl.dtype, 0.02)]
    n_noisy = W.region_counts(wl.segments)[2]
    x = W.make(wl.wid, W.T_LATENT, (n_noisy, hid), "fp32")
    return X, ws, x


@pytest.mark.parametrize("name,steps,checked", [("tiny_fp32", 1, (0,)),
                                                ("policy_bf16", 10, (0, 1, 9))])
def test_denoiser_chain_teacher_forced(name, steps, checked):
    """Every stage of a step is checked against the oracle applied to the
    GPU's own inputs of that stage (teacher forcing), at the per-kernel
    tolerance.  The step's end-to-end velocity is held to the contract
    against the oracle chain with the same storage dtype."""
    dev = device()
    P = _pipeline()
    wl = W.BY_NAME[name]
    X, ws, x = _inputs(wl)
    den = P.DenoiserStep(wl, W.to_torch(X), *(W.to_torch(w) for w in ws), torch.from_numpy(x.f32),
                         device=dev)
    pos, reg, n_ar = olayout.build(wl.segments)
    r0 = den.r_noisy
    h, d = wl.n_heads, wl.head_dim
    Xc = X.f32[:r0]
    wf = [w.f32 for w in ws]
    sig = wl.sigmas
    tol = "bf16" if wl.dtype == "bf16" else "fp32"
    for s in range(steps):
        x_in = to_np(den.x)             # teacher forcing: start from the GPU's x
        X_in = to_np(den.X)             # ... and its packed copy
        if s not in checked:
            den.step(sig[s], sig[s + 1])
            continue
        say("chain %s step %d" % (name, s))
        den.project_qkv()
        torch.cuda.synchronize()
        Y = to_np(den.Y)
        rows = np.r_[0:n_ar + 2, np.random.default_rng(s).choice(den.n, 64)]
        want_y = np.stack([oproj.project_rows(X_in[r:r + 1], wf[0] if r < n_ar else wf[1])[0]
                           for r in rows])
        assert_parity(Y[rows], want_y, tol, "qkv (teacher-forced)")
        den.rope_k()
        den.attention()
        torch.cuda.synchronize()
        y4 = Y.reshape(den.n, 3, h, d)
        qr = omrope.apply(y4[:, 0], pos, wl.sections, wl.theta)
        kr = omrope.apply(y4[:, 1], pos, wl.sections, wl.theta)
        want_o, _ = oattn.attention(qr, kr, y4[:, 2], 0, W.AR_CAUSAL_DM_FULL, n_ar=n_ar)
        O = to_np(den.O).reshape(den.n, h, d)
        assert_parity(O, want_o, tol, "rope+attention (t-f)")
        den.project_o()
        torch.cuda.synchronize()
        Z = to_np(den.Z)
        want_z = oproj.project(O.reshape(den.n, h * d), wf[2], wf[3], n_ar)
        assert_parity(Z, want_z, tol, "o_proj (teacher-forced)")
        den.euler(sig[s], sig[s + 1])
        torch.cuda.synchronize()
        want_x = oeuler.step(x_in, Z[r0:], sig[s], sig[s + 1])
        assert_parity(to_np(den.x), want_x, tol, "euler (teacher-forced)")
        # end to end from the same x: against the chain with the workload's
        # storage dtype (asserted), and against the unrounded chain (reported)
        store = "bf16" if tol == "bf16" else None
        ref = oden.step(x_in, Xc, *wf, pos, n_ar, h, d, wl.sections, wl.theta, sig[s], sig[s + 1],
                        x_as_input=X_in[r0:], store=store)
        assert_parity(Z[r0:], ref["vel"], tol, "end-to-end velocity (%s chain)" % (store or "fp64"))
        if store:
            raw = oden.step(x_in, Xc, *wf, pos, n_ar, h, d, wl.sections, wl.theta, sig[s],
                            sig[s + 1], x_as_input=X_in[r0:])
            ma, rl = errors(Z[r0:], raw["vel"])
            say("  end-to-end velocity vs the unrounded fp64 chain: max_abs=%.3e rel_l2=%.3e" % (ma, rl))


@pytest.mark.parametrize("size", ["stream_chunk_bf16", "mini"])
def test_streaming_rollout_all_chunks_through_the_ring_wrap(size):
    """All chunks x 4 steps of the streaming workload (16 chunks; 11 at the
    reduced size).  From chunk 8 on, each append overwrites a ring slot that
    an earlier appended chunk filled; every call is compared with the
    oracle's rolling cache on sampled rows and heads, and the cache itself
    is compared with the oracle's after every append."""
    dev = device()
    P = _pipeline()
    wl = stream_workload(size)
    h, d = wl.n_heads, wl.head_dim
    ft = wl.stream_views * wl.stream_gh * wl.stream_gw
    slots = wl.stream_history_frames
    n_prefix = wl.stream_text + 2
    assert wl.stream_chunks > slots  # the rollout wraps the ring
    pos, reg, n_ar = olayout.build(wl.segments)
    # the layout of the first chunk: prefix | 8 history frames | chunk frame 8
    pre_k = W.make(3, 50, (n_prefix + slots * ft, h, d), "bf16")
    pre_v = W.make(3, 51, (n_prefix + slots * ft, h, d), "bf16")
    st = P.StreamState(h, d, n_prefix, ft, slots, wl.sections, wl.theta, device=dev)
    st.fill(W.to_torch(pre_k, dev), W.to_torch(pre_v, dev),
            torch.from_numpy(pos[:n_prefix + slots * ft]).to(dev))
    oc = ostream.RollingCache(pre_k.f32[:n_prefix], pre_v.f32[:n_prefix], pos[:n_prefix],
                              pre_k.f32[n_prefix:], pre_v.f32[n_prefix:],
                              pos[n_prefix:n_prefix + slots * ft], ft, wl.sections, wl.theta)
    t0 = n_ar + 15000.0
    chunk_pos = pos[n_prefix + slots * ft:].copy()   # frame 8; later frames shift t
    O = torch.empty((ft, h, d), dtype=torch.bfloat16, device=dev)
    rng = np.random.default_rng(9)
    n_cache = n_prefix + slots * ft
    for c in range(wl.stream_chunks):
        cp = chunk_pos.copy()
        cp[:, 0] = np.float32(t0 + slots + c)
        for s in range(wl.stream_steps):
            q = W.make(3, 60, (ft, h, d), "bf16", 1.0, c, s)
            k = W.make(3, 61, (ft, h, d), "bf16", 1.0, c, s)
            v = W.make(3, 62, (ft, h, d), "bf16", 1.0, c, s)
            Pd = torch.from_numpy(cp).to(dev)
            st.attend(W.to_torch(q, dev), W.to_torch(k, dev), W.to_torch(v, dev), Pd, O)
            torch.cuda.synchronize()
            rows = sorted(set(rng.choice(ft, min(16, ft), replace=False).tolist()) | {0, ft - 1})
            heads = sorted(set(rng.choice(h, min(2, h), replace=False).tolist()) | {h - 1})
            want, kr = oc.attend(q.f32, k.f32, v.f32, cp, rows=rows, heads=heads)
            say("stream chunk %d step %d" % (c, s))
            assert_parity(to_np(O)[rows][:, heads], want, "bf16", "stream c%d s%d" % (c, s))
        st.append(c)
        oc.append(c, kr, v.f32)
        # the slot this chunk went to (from chunk 8 on it held chunk c - 8)
        a = n_prefix + (c % slots) * ft
        assert_parity(to_np(st.K[a:a + ft]), oc.k[a:a + ft], "bf16", "cache K slot %d" % (c % slots))
        np.testing.assert_array_equal(to_np(st.V[a:a + ft]), oc.v[a:a + ft])
    # after the wrap the whole cache holds the latest 8 chunks, rotated
    assert_parity(to_np(st.K[:n_cache]), oc.k, "bf16", "stream cache K")
    np.testing.assert_array_equal(to_np(st.V[:n_cache]), oc.v)


def _sampled_rows(n, n_ar, r0, seed, n_random):
    """All AR rows, 64 rows on each side of the AR/DM and clean/noisy
    boundaries, n_random DM rows and the last row, sorted."""
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([
        np.arange(n_ar), np.arange(n_ar - 64, n_ar + 64), np.arange(r0 - 64, r0 + 64),
        rng.choice(np.arange(n_ar, n), size=n_random, replace=False), [n - 1]]))


def test_long_480p_chain_step_sampled_rows():
    """One chained step of the long 480p workload (76,954 tokens, both rooms'
    3,072 x 9,216 QKV and 3,072 x 3,072 O weights), each stage teacher-forced
    on sampled rows: QKV projection, mRoPE of K, attention with Q rotated on
    load (3 heads), O projection, Euler."""
    dev = device()
    P = _pipeline()
    wl = W.BY_NAME["t2v480p_long_bf16"]
    X, ws, x = _inputs(wl)
    den = P.DenoiserStep(wl, W.to_torch(X), *(W.to_torch(w) for w in ws), torch.from_numpy(x.f32),
                         device=dev)
    del X
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h, d = den.n, wl.n_heads, wl.head_dim
    r0 = den.r_noisy
    wf = [w.f32 for w in ws]
    sig = wl.sigmas
    rows = _sampled_rows(n, n_ar, r0, 31, 256)
    rt = torch.from_numpy(rows).to(dev)
    ar = rows < n_ar
    say("chain long-480p n=%d sampled rows %d" % (n, len(rows)))
    X_in = to_np(den.X.index_select(0, rt))
    den.project_qkv()
    torch.cuda.synchronize()
    Y = to_np(den.Y.index_select(0, rt))
    want_y = np.empty_like(Y, dtype=np.float64)
    want_y[ar] = oproj.project_rows(X_in[ar], wf[0])
    want_y[~ar] = oproj.project_rows(X_in[~ar], wf[1])
    assert_parity(Y, want_y, "bf16", "qkv long-480p")
    heads = [0, 11, 23]
    y4 = den.Y.view(n, 3, h, d)
    ht = torch.tensor(heads, device=dev)
    k_raw = Y.reshape(len(rows), 3, h, d)[:, 1][:, heads]
    den.rope_k()
    den.attention()
    torch.cuda.synchronize()
    kr_all = to_np(y4[:, 1].index_select(1, ht))         # the GPU's rotated K, every key
    assert_parity(kr_all[rows], omrope.apply(k_raw, pos[rows], wl.sections, wl.theta), "bf16",
                  "mrope K long-480p")
    v_all = to_np(y4[:, 2].index_select(1, ht))
    qr = omrope.apply(Y.reshape(len(rows), 3, h, d)[:, 0][:, heads], pos[rows], wl.sections, wl.theta)
    want_o = oattn.attention_rows(qr, kr_all, v_all, rows, [0, 1, 2], 0, W.AR_CAUSAL_DM_FULL,
                                  n_ar=n_ar)
    O = to_np(den.O.index_select(0, rt))
    assert_parity(O.reshape(len(rows), h, d)[:, heads], want_o, "bf16", "attention long-480p")
    den.project_o()
    torch.cuda.synchronize()
    Z = to_np(den.Z.index_select(0, rt))
    want_z = np.empty_like(Z, dtype=np.float64)
    want_z[ar] = oproj.project_rows(O[ar], wf[2])
    want_z[~ar] = oproj.project_rows(O[~ar], wf[3])
    assert_parity(Z, want_z, "bf16", "o_proj long-480p")
    noisy = rows[rows >= r0]
    nt = torch.from_numpy(noisy - r0).to(dev)
    x_in = to_np(den.x.index_select(0, nt))  # the Euler step's input
    den.euler(sig[0], sig[1])
    torch.cuda.synchronize()
    want_x = oeuler.step(x_in, Z[rows >= r0], sig[0], sig[1])
    assert_parity(to_np(den.x.index_select(0, nt)), want_x, "fp32", "euler long-480p")
    # the mirror into the next step's packed input is the bf16 of x
    got_mirror = to_np(den.X.index_select(0, torch.from_numpy(noisy).to(dev)))
    np.testing.assert_array_equal(got_mirror, W.bf16_to_f32(W.bf16_bits(to_np(den.x.index_select(0, nt)))))
