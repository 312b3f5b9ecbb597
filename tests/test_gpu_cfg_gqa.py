"""GPU parity of classifier-free guidance and grouped key/value heads
against the oracle ("Cosmos 3 方法原理全解" §7.2 CFG equation, §7.3
generation loop; §12.4 model table).

* flow_cfg_euler_step: one pass over x, v_cond and v_base; against
  oracle.cfg.euler_step, and bitwise equal to flow_euler_step with v_base at
  w = 0; the bf16 mirror is the RNE of x, bit for bit.
* mot_attention_fwd with a batch: independent items, a shared Q (batch
  stride 0) and overlapping key views, each item against the oracle.
* grouped key/value heads: against the oracle, and bitwise equal to the same
  launch with every key/value head repeated for its group (multi-head).
* GuidedDenoiserStep: both predictions of a guided sampler step in one
  attention launch over [AR cond | DM | AR base], teacher-forced stage by
  stage against the oracle, and end to end against oracle.cfg.step with
  bf16 storage; on the policy workload (full) and on the grouped-head 480p
  workload (sampled rows and heads).
"""
import dataclasses

import numpy as np
import pytest

import workloads as W
from oracle import attention as oattn
from oracle import cfg as ocfg
from oracle import denoiser as oden
from oracle import layout as olayout
from oracle import mrope as omrope
from oracle import projection as oproj
from tests.gpu_util import BF16_LSE_ATOL, assert_parity, assert_parity_stored, device, errors, say, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
AR, CH = W.AR_CAUSAL_DM_FULL, W.CHUNK_CAUSAL_KV


def _mot():
    import multimodal_diffusion_transformer_amd as mot
    return mot


def _pipeline():
    from multimodal_diffusion_transformer_amd import pipeline
    return pipeline


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 7, 8, 4099, 4_423_681])
@pytest.mark.parametrize("vdt", ["bf16", "fp32"])
def test_cfg_euler_parity(n, vdt):
    dev = device()
    mot = _mot()
    say("cfg euler n=%d v=%s" % (n, vdt))
    x0 = W.make(30, 1, (n,), "fp32").f32
    vc = W.make(30, 2, (n,), vdt)
    vb = W.make(30, 3, (n,), vdt)
    for w in (3.0, 6.0):
        x = torch.tensor(x0, device=dev)
        xb = torch.empty(n, dtype=torch.bfloat16, device=dev)
        mot.flow_cfg_euler_step(x, W.to_torch(vc, dev), W.to_torch(vb, dev), w, 0.75, 0.5, x_bf16=xb)
        torch.cuda.synchronize()
        got = to_np(x)
        want = ocfg.euler_step(x0, vc.f32, vb.f32, w, 0.75, 0.5)
        assert_parity(got, want, "fp32", "cfg euler w=%g" % w)
        np.testing.assert_array_equal(_bits(xb), W.bf16_bits(got))


def test_cfg_euler_zero_guidance_is_the_plain_update_with_v_base():
    dev = device()
    mot = _mot()
    n = 100_003
    x0 = W.make(31, 1, (n,), "fp32").f32
    vc = W.to_torch(W.make(31, 2, (n,), "bf16"), dev)
    vb = W.to_torch(W.make(31, 3, (n,), "bf16"), dev)
    a = torch.tensor(x0, device=dev)
    b = torch.tensor(x0, device=dev)
    mot.flow_cfg_euler_step(a, vc, vb, 0.0, 1.0, 0.9)
    mot.flow_euler_step(b, vb, 1.0, 0.9)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------
def _stored(got, want, tol, what):
    """A projection output the kernel stores in the workload's type: bf16
    outputs take the stored-value bound (max(2e-2, one bf16 spacing) per
    element, rel-L2 5e-3), since past |4| a spacing exceeds 2e-2 and two
    stored values, or past |8| a stored and an exact one, can differ by more
    than 2e-2 with both correctly rounded; fp32 outputs the fp32 bound."""
    if tol == "bf16":
        assert_parity_stored(got, want, what)
    else:
        assert_parity(got, want, tol, what)


def _rot_q(x, pos, wl, tol):
    """Q rotated by the oracle as the bf16 kernel uses it: rotated on load
    and held as a bf16 MFMA operand, so rounded to bf16 (the chain's
    storage-point reading); fp32 keeps it unrounded."""
    r = omrope.apply(x, pos, wl.sections, wl.theta)
    return oden.round_bf16(r) if tol == "bf16" else r


def _rand(seed, tid, shape, dtype):
    return W.make(seed, tid, shape, dtype)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
def test_attention_batch_of_independent_items(dtype, d):
    dev = device()
    mot = _mot()
    nb, nq, nk, h, n_ar = 3, 200, 330, 2, 90
    q0 = nk - nq
    say("attention batch %s d=%d" % (dtype, d))
    q = [_rand(32, 10 + b, (nq, h, d), dtype) for b in range(nb)]
    k = [_rand(32, 20 + b, (nk, h, d), dtype) for b in range(nb)]
    v = [_rand(32, 30 + b, (nk, h, d), dtype) for b in range(nb)]
    Q = torch.stack([W.to_torch(t, dev) for t in q])
    K = torch.stack([W.to_torch(t, dev) for t in k])
    V = torch.stack([W.to_torch(t, dev) for t in v])
    O = torch.empty_like(Q)
    L = torch.empty((nb, h, nq), dtype=torch.float32, device=dev)
    mot.mot_attention_fwd(Q, K, V, O, mask=AR, q0=q0, n_ar=n_ar, lse=L)
    torch.cuda.synchronize()
    for b in range(nb):
        want, lse = oattn.attention(q[b].f32, k[b].f32, v[b].f32, q0, AR, n_ar=n_ar)
        assert_parity(to_np(O[b]), want, dtype, "batch item %d" % b)
        np.testing.assert_allclose(to_np(L[b]), lse, atol=BF16_LSE_ATOL if dtype == "bf16" else 1e-4, rtol=0)


def test_attention_batch_shared_q_and_overlapping_keys():
    """The guided step's layout in miniature: one buffer [A | S | B] of
    keys; item 0 reads [A | S], item 1 reads [S | B]; Q is shared."""
    dev = device()
    mot = _mot()
    n_ar, n_s, h, d = 70, 250, 2, 128
    n = n_ar + n_s
    say("attention batch shared Q, overlapping keys")
    kbuf = _rand(33, 1, (n + n_ar, h, d), "bf16")
    vbuf = _rand(33, 2, (n + n_ar, h, d), "bf16")
    q = _rand(33, 3, (n_s, h, d), "bf16")
    KB, VB = W.to_torch(kbuf, dev), W.to_torch(vbuf, dev)
    st = KB.stride(0)
    K = torch.as_strided(KB, (2, n, h, d), (n_ar * st, st, d, 1))
    V = torch.as_strided(VB, (2, n, h, d), (n_ar * st, st, d, 1))
    Q = W.to_torch(q, dev).unsqueeze(0).expand(2, n_s, h, d)
    O = torch.empty((2, n_s, h, d), dtype=torch.bfloat16, device=dev)
    mot.mot_attention_fwd(Q, K, V, O, mask=AR, q0=n_ar, n_ar=n_ar)
    torch.cuda.synchronize()
    for b in range(2):
        want, _ = oattn.attention(q.f32, kbuf.f32[b * n_ar:b * n_ar + n], vbuf.f32[b * n_ar:b * n_ar + n],
                                  n_ar, AR, n_ar=n_ar)
        assert_parity(to_np(O[b]), want, "bf16", "shared-Q item %d" % b)


GQA_CASES = [
    # dtype, d, H, H_kv, nq, nk, q0, mode
    ("bf16", 128, 8, 2, 300, 300, 0, AR),
    ("bf16", 128, 32, 8, 200, 260, 60, AR),
    ("bf16", 64, 6, 3, 257, 257, 0, AR),
    ("bf16", 128, 16, 8, 2 * 45 + 7, 33 + 2 * 45 + 7, 33, CH),
    ("fp32", 64, 4, 1, 150, 150, 0, AR),
    ("fp32", 128, 4, 2, 97, 130, 33, CH),
    ("bf16", 80, 64, 8, 200, 260, 60, AR),    # the model table's largest head shape
    ("bf16", 80, 8, 2, 2 * 45 + 7, 33 + 2 * 45 + 7, 33, CH),
    ("fp32", 80, 4, 2, 150, 150, 0, AR),
]


@pytest.mark.parametrize("case", GQA_CASES, ids=lambda c: "%s_d%d_h%d_kv%d_%s" % (
    c[0], c[1], c[2], c[3], "ar" if c[7] == AR else "chunk"))
def test_attention_grouped_heads(case):
    dtype, d, h, hk, nq, nk, q0, mode = case
    dev = device()
    mot = _mot()
    say("attention GQA %s d=%d %d/%d heads" % (dtype, d, h, hk))
    kw = dict(n_ar=min(nk, 100)) if mode == AR else dict(n_prefix=33, chunk_len=45)
    q = _rand(34, 1, (nq, h, d), dtype)
    k = _rand(34, 2, (nk, hk, d), dtype)
    v = _rand(34, 3, (nk, hk, d), dtype)
    Q, K, V = W.to_torch(q, dev), W.to_torch(k, dev), W.to_torch(v, dev)
    O = torch.empty((nq, h, d), dtype=Q.dtype, device=dev)
    mot.mot_attention_fwd(Q, K, V, O, mask=mode, q0=q0, **kw)
    # the same launch with every key/value head repeated for its group
    Kr = K.repeat_interleave(h // hk, dim=1).contiguous()
    Vr = V.repeat_interleave(h // hk, dim=1).contiguous()
    O2 = torch.empty_like(O)
    mot.mot_attention_fwd(Q, Kr, Vr, O2, mask=mode, q0=q0, **kw)
    torch.cuda.synchronize()
    want, _ = oattn.attention(q.f32, k.f32, v.f32, q0, mode, **kw)
    assert_parity(to_np(O), want, dtype, "GQA %d/%d" % (h, hk))
    assert torch.equal(O.view(torch.int16) if dtype == "bf16" else O,
                       O2.view(torch.int16) if dtype == "bf16" else O2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_mrope_at_head_size_80(dtype):
    """Standalone mRoPE at the Super head size (40 pairs in t / h / w
    sections of 10 / 15 / 15; 25 tokens per workgroup, the last lanes idle)
    on the K view of a packed [N, 64 + 16, 80] projection output."""
    dev = device()
    mot = _mot()
    wl = W.BY_NAME["super_t2v480p_bf16"]
    pos, reg, n_ar = olayout.build(W.BY_NAME["policy_bf16"].segments)
    n, h, hk, d = len(reg), wl.n_heads, wl.kv_heads, wl.head_dim
    y = _rand(38, 1, (n, h + 2 * hk, d), dtype)
    Y = W.to_torch(y, dev).contiguous()
    mot.mrope_apply(Y[:, h:h + hk], torch.from_numpy(pos).to(dev), wl.sections, wl.theta)
    torch.cuda.synchronize()
    got = to_np(Y)
    assert_parity(got[:, h:h + hk], omrope.apply(y.f32[:, h:h + hk], pos, wl.sections, wl.theta), dtype,
                  "mrope D = 80")
    np.testing.assert_array_equal(got[:, :h], y.f32[:, :h])
    np.testing.assert_array_equal(got[:, h + hk:], y.f32[:, h + hk:])


@pytest.mark.parametrize("mode", [AR, CH], ids=["ar", "chunk"])
def test_attention_d80_is_d128_on_zero_padded_heads(mode):
    """Head size 80 (the model table's Super heads) runs the D = 128
    kernel's arithmetic on 80 dims: at the same scale, its O and LSE equal
    the D = 128 kernel's on the same heads zero-padded to 128 dims, bit for
    bit."""
    dev = device()
    mot = _mot()
    nq, nk, q0, h, hk = 700, 1201, 501, 64, 8
    kw = dict(n_ar=300) if mode == AR else dict(n_prefix=258, chunk_len=240)
    say("attention D = 80 vs zero-padded D = 128, %s" % ("ar" if mode == AR else "chunk"))
    q = W.to_torch(_rand(37, 1, (nq, h, 80), "bf16"), dev)
    k = W.to_torch(_rand(37, 2, (nk, hk, 80), "bf16"), dev)
    v = W.to_torch(_rand(37, 3, (nk, hk, 80), "bf16"), dev)
    outs = []
    for d in (80, 128):
        pad = lambda t: torch.nn.functional.pad(t, (0, d - 80)).contiguous()
        O = torch.empty((nq, h, d), dtype=torch.bfloat16, device=dev)
        L = torch.empty((h, nq), dtype=torch.float32, device=dev)
        mot.mot_attention_fwd(pad(q), pad(k), pad(v), O, mask=mode, q0=q0, lse=L, scale=1.0 / 80 ** 0.5, **kw)
        outs.append((O[..., :80].contiguous(), L))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))


@pytest.mark.parametrize("name", ["nano_t2v480p_bf16", "super_t2v480p_bf16"])
def test_attention_grouped_heads_480p_sampled_rows(name):
    """The grouped-head 480p workloads (32 / 8 heads of 128 and 64 / 8 heads
    of 80, 25,474 tokens): K and V strided views of the fused
    [N, (H + 2 H_kv) D] projection output, Q rotated on load; sampled rows of
    4 heads spanning 2 key/value heads."""
    dev = device()
    mot = _mot()
    wl = W.BY_NAME[name]
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h, hk, d = len(reg), wl.n_heads, wl.kv_heads, wl.head_dim
    say("attention GQA 480p n=%d %d/%d heads" % (n, h, hk))
    q = _rand(35, W.T_Q, (n, h, d), "bf16")
    k = _rand(35, W.T_K, (n, hk, d), "bf16")
    v = _rand(35, W.T_V, (n, hk, d), "bf16")
    Y = torch.empty((n, (h + 2 * hk) * d), dtype=torch.bfloat16, device=dev)
    Y[:, :h * d] = W.to_torch(q, dev).view(n, h * d)
    Y[:, h * d:(h + hk) * d] = W.to_torch(k, dev).view(n, hk * d)
    Y[:, (h + hk) * d:] = W.to_torch(v, dev).view(n, hk * d)
    O = torch.empty((n, h, d), dtype=torch.bfloat16, device=dev)
    mot.mot_attention_fwd(Y[:, :h * d].view(n, h, d), Y[:, h * d:(h + hk) * d].view(n, hk, d),
                          Y[:, (h + hk) * d:].view(n, hk, d), O, mask=AR, n_ar=n_ar,
                          q_pos=torch.from_numpy(pos).to(dev), sections=wl.sections, theta=wl.theta)
    torch.cuda.synchronize()
    rng = np.random.default_rng(35)
    rows = np.unique(np.concatenate([np.arange(n_ar), np.arange(n_ar, n_ar + 64),
                                     rng.choice(np.arange(n_ar, n), 64, replace=False), [n - 1]]))
    heads = [0, 3, h // hk, h - 1]
    kvh = [oattn.kv_head(x, h, hk) for x in heads]
    got = to_np(O.index_select(0, torch.from_numpy(rows).to(dev)))[:, heads]
    qr = omrope.apply(q.f32[rows], pos[rows], wl.sections, wl.theta)
    want = oattn.attention_rows(qr, k.f32, v.f32, rows, heads, 0, AR, n_ar=n_ar, kv_heads=kvh)
    assert_parity(got, want, "bf16", "GQA 480p sampled")


# ---------------------------------------------------------------------------
def _guided_inputs(wl):
    n = wl.n_tokens
    hid, h, d, hk = wl.hidden, wl.n_heads, wl.head_dim, wl.kv_heads
    n_ar, n_clean, n_noisy = W.region_counts(wl.segments)
    width = (h + 2 * hk) * d
    X = W.make(wl.wid, W.T_X, (n, hid), wl.dtype)
    Xb = W.make(wl.wid, W.T_X_BASE, (n_ar, hid), wl.dtype)
    ws = [W.make(wl.wid, W.T_WQKV_AR, (hid, width), wl.dtype, 0.02),
          W.make(wl.wid, W.T_WQKV_DM, (hid, width), wl.dtype, 0.02),
          W.make(wl.wid, W.T_WO_AR, (h * d, hid), wl.dtype, 0.02),
          W.make(wl.wid, W.T_WO_DM, (h * d, hid), wl.dtype, 0.02)]
    x = W.make(wl.wid, W.T_LATENT, (n_noisy, hid), "fp32")
    return X, Xb, ws, x


def _guided_step(wl, guidance, dev):
    P = _pipeline()
    X, Xb, ws, x = _guided_inputs(wl)
    n_ar, n_clean, _ = W.region_counts(wl.segments)
    g = P.GuidedDenoiserStep(wl, W.to_torch(X)[:n_ar], W.to_torch(Xb), W.to_torch(X)[n_ar:n_ar + n_clean],
                             *(W.to_torch(w) for w in ws), torch.from_numpy(x.f32), guidance, device=dev)
    return g, X, Xb, ws, x


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,guidance,steps,checked", [("policy_bf16", 3.0, 10, (0, 1, 9)),
                                                         ("tiny_fp32", 6.0, 1, (0,)),
                                                         ("super_on_policy_bf16", 3.0, 2, (0, 1))])
def test_guided_step_teacher_forced(name, guidance, steps, checked):
    """super_on_policy_bf16: the model table's Super heads (64 / 8 of 80,
    hidden 5120) on the policy layout."""
    dev = device()
    if name == "super_on_policy_bf16":
        wl = dataclasses.replace(W.BY_NAME["super_t2v480p_bf16"], name=name,
                                 segments=W.BY_NAME["policy_bf16"].segments, sigmas=W.BY_NAME["policy_bf16"].sigmas)
    else:
        wl = W.BY_NAME[name]
    g, X, Xb, ws, x = _guided_step(wl, guidance, dev)
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h, d, hk = g.n, wl.n_heads, wl.head_dim, wl.kv_heads
    n_dm, c = g.n_dm, g.n_clean
    wf = [w.f32 for w in ws]
    sig = wl.sigmas
    tol = "bf16" if wl.dtype == "bf16" else "fp32"
    Xc_ar, Xb_ar, X_clean = X.f32[:n_ar], Xb.f32, X.f32[n_ar:n_ar + c]
    # the request's cached prompts: AR rows through the Reasoner weights,
    # keys rotated at the AR positions (against the chain with the
    # workload's storage: the projection is stored before the rotation)
    torch.cuda.synchronize()
    QKV = to_np(g.QKV)
    for name_, X_ar, rows in (("cond", Xc_ar, slice(0, n_ar)), ("base", Xb_ar, slice(n_ar + n_dm, None))):
        y = oproj.project_rows(X_ar, wf[0])
        if tol == "bf16":
            y = oden.round_bf16(y)
        q_, k_, v_ = oproj.split_qkv(y, h, d, hk)
        got = QKV[rows]
        _stored(got[:, h * d:(h + hk) * d].reshape(n_ar, hk, d),
                      omrope.apply(k_, pos[:n_ar], wl.sections, wl.theta), tol, "AR %s K" % name_)
        _stored(got[:, (h + hk) * d:], v_.reshape(n_ar, -1), tol, "AR %s V" % name_)
    for s in range(steps):
        x_in = to_np(g.x)
        Xdm_in = to_np(g.Xdm)
        if s not in checked:
            g.step(sig[s], sig[s + 1])
            continue
        say("guided %s step %d (w=%g)" % (name, s, guidance))
        g.project_qkv()
        torch.cuda.synchronize()
        Ydm = to_np(g.Ydm)
        _stored(Ydm, oproj.project_rows(Xdm_in, wf[1]), tol, "qkv DM rows")
        g.rope_k()
        g.attention()
        torch.cuda.synchronize()
        QKV = to_np(g.QKV)
        q_dm = _rot_q(Ydm[:, :h * d].reshape(n_dm, h, d), pos[n_ar:], wl, tol)
        Kall = QKV[:, h * d:(h + hk) * d].reshape(-1, hk, d)    # rotated keys, all rows
        Vall = QKV[:, (h + hk) * d:].reshape(-1, hk, d)
        O = to_np(g.O).reshape(2, n_dm, h, d)
        for b in range(2):
            want, _ = oattn.attention(q_dm, Kall[b * n_ar:b * n_ar + n], Vall[b * n_ar:b * n_ar + n],
                                      n_ar, AR, n_ar=n_ar)
            assert_parity(O[b], want, tol, "attention branch %d (t-f)" % b)
        g.project_o()
        torch.cuda.synchronize()
        Z = to_np(g.Z)
        for b in range(2):
            assert_parity(Z[b], oproj.project_rows(O[b].reshape(n_dm, h * d), wf[3]), tol,
                          "o_proj branch %d (t-f)" % b)
        g.euler(sig[s], sig[s + 1])
        torch.cuda.synchronize()
        want_x = ocfg.euler_step(x_in, Z[0, c:], Z[1, c:], guidance, sig[s], sig[s + 1])
        assert_parity(to_np(g.x), want_x, "fp32", "cfg euler (t-f)")
        # end to end from the same x against the oracle's guided step
        store = "bf16" if tol == "bf16" else None
        ref = ocfg.step(x_in, Xc_ar, Xb_ar, X_clean, *wf, pos, n_ar, h, d, wl.sections, wl.theta,
                        guidance, sig[s], sig[s + 1], x_as_input=Xdm_in[c:], store=store,
                        n_kv_heads=hk)
        # each prediction at the contract; the guided velocity within the
        # contract carried through the combination (its error is at most
        # |1 - w| err(v_base) + |w| err(v_cond)); the updated latent at the
        # contract
        for b, key in ((0, "vel_cond"), (1, "vel_base")):
            assert_parity(Z[b, c:], ref[key], tol, "end-to-end %s" % key)
        v_gpu = ocfg.combine(Z[0, c:], Z[1, c:], guidance)
        ma, rl = errors(v_gpu, ref["vel"])
        say("  end-to-end guided velocity: max_abs=%.3e rel_l2=%.3e" % (ma, rl))
        lim_a, lim_r = (2e-2, 5e-3) if tol == "bf16" else (1e-4, 1e-5)
        wc, wb = abs(guidance), abs(1.0 - guidance)
        nrm = lambda t: float(np.linalg.norm(np.asarray(t, np.float64)))
        assert ma <= (wb + wc) * lim_a
        assert rl * nrm(ref["vel"]) <= lim_r * (wb * nrm(ref["vel_base"]) + wc * nrm(ref["vel_cond"]))
        assert_parity(to_np(g.x), ref["x_next"], "fp32" if tol == "fp32" else "bf16",
                      "end-to-end x_next")


@pytest.mark.parametrize("name", ["nano_t2v480p_bf16", "super_t2v480p_bf16"])
def test_guided_step_grouped_heads_480p_sampled(name):
    """The grouped-head 480p workloads with guidance 6: one guided step,
    each stage teacher-forced on sampled rows and heads."""
    dev = device()
    wl = W.BY_NAME[name]
    g, X, Xb, ws, x = _guided_step(wl, wl.guidance, dev)
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h, d, hk = g.n, wl.n_heads, wl.head_dim, wl.kv_heads
    n_dm, c = g.n_dm, g.n_clean
    wf = [w.f32 for w in ws]
    sig = wl.sigmas
    say("guided GQA 480p n=%d, %d/%d heads, w=%g" % (n, h, hk, wl.guidance))
    rng = np.random.default_rng(36)
    rows = np.unique(np.concatenate([np.arange(64), rng.choice(n_dm, 192, replace=False), [n_dm - 1]]))
    rt = torch.from_numpy(rows).to(dev)
    Xdm_in = to_np(g.Xdm.index_select(0, rt))
    g.project_qkv()
    torch.cuda.synchronize()
    Ydm = to_np(g.Ydm.index_select(0, rt))
    _stored(Ydm, oproj.project_rows(Xdm_in, wf[1]), "bf16", "qkv DM rows (sampled)")
    g.rope_k()
    g.attention()
    torch.cuda.synchronize()
    heads = [0, 5, 30]
    kv = sorted({oattn.kv_head(x_, h, hk) for x_ in heads})
    kvh = [kv.index(oattn.kv_head(x_, h, hk)) for x_ in heads]
    K3 = g.QKV[:, h * d:(h + hk) * d].view(-1, hk, d)
    V3 = g.QKV[:, (h + hk) * d:].view(-1, hk, d)
    kt = torch.tensor(kv, device=dev)
    Kall, Vall = to_np(K3.index_select(1, kt)), to_np(V3.index_select(1, kt))
    q_dm = _rot_q(Ydm[:, :h * d].reshape(len(rows), h, d)[:, heads], pos[n_ar + rows], wl, "bf16")
    O = to_np(g.O.index_select(1, rt)).reshape(2, len(rows), h, d)
    for b in range(2):
        want = oattn.attention_rows(q_dm, Kall[b * n_ar:b * n_ar + n], Vall[b * n_ar:b * n_ar + n],
                                    n_ar + rows, [0, 1, 2], 0, AR, n_ar=n_ar, kv_heads=kvh)
        assert_parity(O[b][:, heads], want, "bf16", "attention branch %d (sampled)" % b)
    g.project_o()
    torch.cuda.synchronize()
    Z = to_np(g.Z.index_select(1, rt))
    for b in range(2):
        assert_parity(Z[b], oproj.project_rows(O[b].reshape(len(rows), h * d), wf[3]), "bf16",
                      "o_proj branch %d (sampled)" % b)
    noisy = rows[rows >= c]
    nt = torch.from_numpy(noisy - c).to(dev)
    x_in = to_np(g.x.index_select(0, nt))  # the Euler step's input
    g.euler(sig[0], sig[1])
    torch.cuda.synchronize()
    sel = rows >= c
    want_x = ocfg.euler_step(x_in, Z[0][sel], Z[1][sel], wl.guidance, sig[0], sig[1])
    assert_parity(to_np(g.x.index_select(0, nt)), want_x, "fp32", "cfg euler (sampled)")
