"""GPU parity of the chained one-layer denoiser step (projection -> mRoPE ->
attention -> output projection -> Euler) and of the streaming rollout,
teacher-forced step by step against the oracle."""
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
from tests.gpu_util import assert_parity, device, errors, say, to_np

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
    tolerance.  The step's end-to-end velocity against an unrounded fp64
    chain is reported, and bounded loosely: it composes four bf16 stores."""
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
        # end to end from the same x, against the unrounded fp64 chain
        ref = oden.step(x_in, Xc, *wf, pos, n_ar, h, d, wl.sections, wl.theta, sig[s], sig[s + 1],
                        x_as_input=X_in[r0:])
        ma, rl = errors(Z[r0:], ref["vel"])
        say("  end-to-end velocity vs fp64 chain: max_abs=%.3e rel_l2=%.3e" % (ma, rl))
        assert rl < (2e-2 if tol == "bf16" else 1e-4)


def test_streaming_rollout_sampled():
    dev = device()
    P = _pipeline()
    wl = W.BY_NAME["stream_chunk_bf16"]
    h, d = wl.n_heads, wl.head_dim
    ft = wl.stream_views * wl.stream_gh * wl.stream_gw
    slots = wl.stream_history_frames
    n_prefix = wl.stream_text + 2
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
    n_chunks = 3  # the bench rolls all 16; parity samples the first three
    for c in range(n_chunks):
        cp = chunk_pos.copy()
        cp[:, 0] = np.float32(t0 + slots + c)
        for s in range(wl.stream_steps):
            q = W.make(3, 60, (ft, h, d), "bf16", 1.0, c, s)
            k = W.make(3, 61, (ft, h, d), "bf16", 1.0, c, s)
            v = W.make(3, 62, (ft, h, d), "bf16", 1.0, c, s)
            Pd = torch.from_numpy(cp).to(dev)
            st.attend(W.to_torch(q, dev), W.to_torch(k, dev), W.to_torch(v, dev), Pd, O)
            torch.cuda.synchronize()
            rows = sorted(rng.choice(ft, 24, replace=False).tolist())
            heads = [0, 11, 23]
            want, kr = oc.attend(q.f32, k.f32, v.f32, cp, rows=rows, heads=heads)
            say("stream chunk %d step %d" % (c, s))
            assert_parity(to_np(O)[rows][:, heads], want, "bf16", "stream")
        st.append(c)
        oc.append(c, kr, v.f32)
    # the cache holds the rotated keys of the appended chunks
    got_k = to_np(st.K[:n_prefix + slots * ft])
    assert_parity(got_k, oc.k, "bf16", "stream cache K")
