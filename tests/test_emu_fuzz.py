"""Randomised parity of the kernels on the CPU SIMT emulator (see
tests/test_emu_kernels.py): hypothesis draws valid problems (shapes, ragged
sizes, masks, query offsets, grouped heads, batches, padded strides, input
and softmax scales, mRoPE sections and positions, guidance weights and
noise levels, scheduling modes) and each is compared with the oracle at the
GPU tests' tolerances.  Derandomised, so every run draws the same examples.
"""
import ctypes
import math
import os

import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import workloads as W  # noqa: E402
from oracle import attention as oattn  # noqa: E402
from oracle import block as oblock  # noqa: E402
from oracle import cfg as ocfg  # noqa: E402
from oracle import euler as oeuler  # noqa: E402
from oracle import denoiser as odenoiser  # noqa: E402
from oracle import mrope as omrope  # noqa: E402
from oracle import projection as oproj  # noqa: E402
from tests import emu_lib  # noqa: E402
from tests.gpu_util import BF16_LSE_ATOL, assert_parity, assert_parity_stored, bf16_spacing  # noqa: E402
from tests.test_emu_kernels import BF16, FP32, _el, attention, bits_of, region_linear, val  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(emu_lib.CXX), reason="host clang++ missing")
AR, CH = W.AR_CAUSAL_DM_FULL, W.CHUNK_CAUSAL_KV
SETTINGS = dict(deadline=None, derandomize=True, suppress_health_check=list(HealthCheck), database=None)
# MOT_FUZZ_SCALE=k draws k times as many examples (a longer run by hand)
SCALE = int(os.environ.get("MOT_FUZZ_SCALE", "1"))


@pytest.fixture(scope="module")
def E(tmp_path_factory):
    pytest.importorskip("multimodal_diffusion_transformer_amd._binding")
    e = emu_lib.Emu(emu_lib.build(str(tmp_path_factory.mktemp("emu_fuzz"))))
    yield e
    e.free_all()


@st.composite
def attn_problem(draw):
    d = draw(st.sampled_from([64, 80, 128]))
    hk = draw(st.integers(1, 4))
    h = hk * draw(st.integers(1, 4))
    mask = draw(st.sampled_from([AR, CH]))
    nq = draw(st.integers(1, 260))
    if mask == AR:
        q0 = draw(st.integers(0, 150))
        nk = q0 + nq + draw(st.integers(0, 90))
        n_ar = draw(st.integers(0, nk))
        n_prefix, cl = 0, 0
    else:
        n_prefix = draw(st.integers(0, 130))
        q0 = n_prefix + draw(st.integers(0, 70))
        cl = draw(st.integers(1, 160))
        nk = draw(st.integers(max(n_prefix, 1), q0 + nq + 40))
        n_ar = 0
    return dict(d=d, h=h, hk=hk, mask=mask, nq=nq, nk=nk, q0=q0, n_ar=n_ar, n_prefix=n_prefix, cl=cl,
                batch=draw(st.integers(1, 2)), pad=draw(st.integers(0, 2)),
                # (input std, softmax scale; 0 = 1/sqrt(D)): score std up to
                # about 4, the regime of the bf16 contract (the workloads'
                # N(0, 1) inputs at 1/sqrt(D) give 1; far more peaked rows
                # make bf16 P alone move O by ~2e-2)
                **dict(zip(("std", "scale"), draw(st.sampled_from(
                    [(0.5, 0.0), (1.0, 0.0), (2.0, 0.0), (0.5, 0.04), (1.0, 0.04), (0.5, 0.3), (1.0, 0.3)])))),
                rope=draw(st.booleans()),
                mode=draw(st.sampled_from([(False, False), (True, True), (True, False), (True, 2)])),
                seed=draw(st.integers(0, 10 ** 6)))


@settings(max_examples=40 * SCALE, **SETTINGS)
@given(pr=attn_problem())
def test_attention_bf16_random_problems(E, pr):
    d, h, hk, nq, nk, B, pad = pr["d"], pr["h"], pr["hk"], pr["nq"], pr["nk"], pr["batch"], pr["pad"]
    E.config(*pr["mode"])
    r = np.random.default_rng(pr["seed"])
    try:
        # padded head dimension: every view has a row stride larger than its heads
        Qb = E.empty((B, nq, h + pad, d), np.uint16)
        Kb = E.empty((B, nk, hk + pad, d), np.uint16)
        Vb = E.empty((B, nk, hk + pad, d), np.uint16)
        Ob = E.empty((B, nq, h + pad, d), np.uint16)
        L = E.empty((B, h, nq), np.float32)
        q = bits_of(r.standard_normal((B, nq, h, d)) * pr["std"])
        k = bits_of(r.standard_normal((B, nk, hk, d)) * pr["std"])
        v = bits_of(r.standard_normal((B, nk, hk, d)))
        Qb[:, :, :h], Kb[:, :, :hk], Vb[:, :, :hk] = q, k, v
        kw = dict(mode=pr["mask"], q0=pr["q0"], n_ar=pr["n_ar"], n_prefix=pr["n_prefix"], chunk_len=pr["cl"],
                  scale=pr["scale"])
        pos, secs = None, (d // 8, 3 * d // 16, 3 * d // 16)
        if pr["rope"]:
            pos = E.array(np.floor(r.uniform(0, 2e4, (nq, 3))).astype(np.float32))
            kw.update(q_pos=pos, sections=secs, theta=1e4)
        views = [t[:, :, :n] for t, n in ((Qb, h), (Kb, hk), (Vb, hk), (Ob, h))]
        if B == 1:
            views = [t[0] for t in views]
            attention(E, *views, lse=L[0], **kw)
        else:
            attention(E, *views, lse=L, **kw)
        for b in range(B):
            qf = val(q[b])
            lse_tol = BF16_LSE_ATOL
            if pr["rope"]:
                # The kernel stores the rotated Q in bf16 (its MFMA operand).
                # Its fp32 rotation and the oracle's fp64 one may round an
                # element to neighbouring bf16 values (one spacing apart),
                # which moves a score by up to scale * sum_d spacing_d |k_d|.
                qf = odenoiser.round_bf16(omrope.apply(qf, np.asarray(pos), secs, 1e4))
                sc = float(np.float32(pr["scale"])) if pr["scale"] else 1.0 / math.sqrt(d)
                kmax = np.abs(val(k[b])).max(axis=0)                       # [hk, d]
                flip = sc * (bf16_spacing(qf) * kmax[np.arange(h) // (h // hk)][None]).sum(-1)  # [nq, h]
                lse_tol = BF16_LSE_ATOL + flip.T
            want, lse = oattn.attention(qf, val(k[b]), val(v[b]), pr["q0"], pr["mask"], pr["n_ar"],
                                        pr["n_prefix"], max(pr["cl"], 1),
                                        scale=float(np.float32(pr["scale"])) if pr["scale"] else None)
            assert_parity(val(Ob[b, :, :h]), want, "bf16", "item %d" % b)
            assert (np.abs(L[b] - lse) <= lse_tol).all(), np.abs(L[b] - lse).max()
            assert (Ob[b, :, h:] == 0).all()  # pad heads untouched
    finally:
        E.free_all()


@settings(max_examples=15 * SCALE, **SETTINGS)
@given(d=st.sampled_from([64, 80, 128]), hk=st.integers(1, 3), g=st.integers(1, 3), nq=st.integers(1, 120),
       extra=st.integers(0, 60), n_ar_frac=st.floats(0, 1), seed=st.integers(0, 10 ** 6))
def test_attention_fp32_random_problems(E, d, hk, g, nq, extra, n_ar_frac, seed):
    E.config(False, True)
    h, nk = hk * g, nq + extra
    n_ar = int(n_ar_frac * nk)
    r = np.random.default_rng(seed)
    try:
        q = r.standard_normal((nq, h, d)).astype(np.float32)
        k = r.standard_normal((nk, hk, d)).astype(np.float32)
        v = r.standard_normal((nk, hk, d)).astype(np.float32)
        O, L = E.empty((nq, h, d), np.float32), E.empty((h, nq), np.float32)
        attention(E, E.array(q), E.array(k), E.array(v), O, mode=AR, q0=extra, n_ar=n_ar, lse=L)
        want, lse = oattn.attention(q, k, v, extra, AR, n_ar)
        assert_parity(O, want, "fp32", "fp32 attention")
        np.testing.assert_allclose(L, lse, atol=1e-4, rtol=0)
    finally:
        E.free_all()


@settings(max_examples=25 * SCALE, **SETTINGS)
@given(n=st.integers(1, 400), ar_frac=st.floats(0, 1), kb=st.integers(1, 5), nb=st.integers(1, 7),
       out_dt=st.sampled_from([BF16, FP32]), epi=st.sampled_from([0, 1, 2]),
       mode=st.sampled_from([(False, False), (True, True), (True, 2)]), seed=st.integers(0, 10 ** 6))
def test_region_linear_bf16_random_problems(E, n, ar_frac, kb, nb, out_dt, epi, mode, seed):
    E.config(*mode)
    K, N = 64 * kb, 64 * nb
    n_ar = int(ar_frac * n)
    r = np.random.default_rng(seed)
    try:
        x = bits_of(r.standard_normal((n, K)))
        wa = bits_of(r.standard_normal((K, N)) / math.sqrt(K))
        wd = bits_of(r.standard_normal((K, N)) / math.sqrt(K))
        want = oproj.project(val(x), val(wa), val(wd), n_ar)
        R = None
        Y = E.empty((n, N), np.uint16 if out_dt == BF16 else np.float32)
        if epi == 1:
            want = oblock.gelu(want)
        elif epi == 2:
            res = r.standard_normal((n, N)) * 3
            res = bits_of(res) if out_dt == BF16 else res.astype(np.float32)
            Y[...] = res
            R = Y
            want = want + (val(res) if out_dt == BF16 else res)
        region_linear(E, E.array(x), E.array(wa) if n_ar > 0 else None, E.array(wd) if n_ar < n else None,
                      Y, n_ar, BF16, out_dt, epi, R)
        got = val(Y) if out_dt == BF16 else Y
        if out_dt == BF16:
            assert_parity_stored(got, want, "gemm")
        else:
            assert_parity(got, want, "bf16", "gemm")
    finally:
        E.free_all()


@settings(max_examples=20 * SCALE, **SETTINGS)
@given(hidden8=st.integers(1, 1024), n=st.integers(1, 12), ar_frac=st.floats(0, 1),
       in_bf16=st.booleans(), out_bf16=st.booleans(), scale=st.sampled_from([0.01, 1.0, 100.0]),
       seed=st.integers(0, 10 ** 6))
def test_layernorm_random_problems(E, hidden8, n, ar_frac, in_bf16, out_bf16, scale, seed):
    E.config(False, False)
    hidden, n_ar = 8 * hidden8, int(ar_frac * n)
    r = np.random.default_rng(seed)
    try:
        x = (r.standard_normal((n, hidden)) * scale + r.standard_normal((n, 1)) * scale).astype(np.float32)
        x = val(bits_of(x)) if in_bf16 else x
        g = [(1 + 0.1 * r.standard_normal(hidden)).astype(np.float32) for _ in range(2)]
        b = [(0.1 * r.standard_normal(hidden)).astype(np.float32) for _ in range(2)]
        X = E.array(bits_of(x) if in_bf16 else x)
        Y = E.empty((n, hidden), np.uint16 if out_bf16 else np.float32)
        ptrs = [emu_lib.ptr(E.array(t)) for t in (g[0], b[0], g[1], b[1])]
        st_ = E.call("mot_layernorm_region", emu_lib.ptr(X), emu_lib.ptr(Y), n, n_ar, hidden, *ptrs,
                     ctypes.c_float(1e-6), BF16 if in_bf16 else FP32, BF16 if out_bf16 else FP32, None)
        assert st_ == 0
        want = oblock.region_layer_norm(x, (g[0], b[0]), (g[1], b[1]), n_ar, 1e-6)
        assert_parity(val(Y) if out_bf16 else Y, want, "bf16" if out_bf16 else "fp32", "layernorm")
    finally:
        E.free_all()


@settings(max_examples=20 * SCALE, **SETTINGS)
@given(parts=st.integers(1, 16), nq=st.integers(1, 60), h=st.integers(1, 5), d=st.sampled_from([64, 80, 128]),
       bf16=st.booleans(), empty_frac=st.floats(0, 0.5), seed=st.integers(0, 10 ** 6))
def test_merge_random_problems(E, parts, nq, h, d, bf16, empty_frac, seed):
    E.config(False, False)
    r = np.random.default_rng(seed)
    try:
        o = r.standard_normal((parts, nq, h, d)).astype(np.float32)
        o = val(bits_of(o)) if bf16 else o
        lse = (r.standard_normal((parts, h, nq)) * 4).astype(np.float32)
        # parts with no key for a row; part 0 always has one
        lse[1:][r.random((parts - 1, h, nq)) < empty_frac] = -np.inf
        Op = E.array(bits_of(o) if bf16 else o)
        Lp = E.array(lse)
        O = E.empty((nq, h, d), np.uint16 if bf16 else np.float32)
        L = E.empty((h, nq), np.float32)
        el = _el(Op)
        st_ = E.call("mot_attention_merge", emu_lib.ptr(Op), emu_lib.ptr(Lp), parts, el[0], nq, h, d, el[1],
                     el[2], emu_lib.ptr(O), h * d, d, emu_lib.ptr(L), BF16 if bf16 else FP32, None)
        assert st_ == 0
        want, wl = oattn.merge(o, lse)
        assert_parity(val(O) if bf16 else O, want, "bf16" if bf16 else "fp32", "merge")
        np.testing.assert_allclose(L, wl, atol=1e-5, rtol=1e-6)
    finally:
        E.free_all()


@settings(max_examples=20, **SETTINGS)
@given(n=st.integers(1, 300), h=st.integers(1, 6), d=st.sampled_from([64, 80, 128]), bf16=st.booleans(),
       cut=st.tuples(st.integers(0, 64), st.integers(0, 64)), pad=st.integers(0, 3),
       pmax=st.sampled_from([10.0, 2e4]), theta=st.sampled_from([1e4, 5e5]), seed=st.integers(0, 10 ** 6))
def test_mrope_random_problems(E, n, h, d, bf16, cut, pad, pmax, theta, seed):
    """Standalone mRoPE on a padded [N, H, D] view: any split of the D/2
    pairs into t / h / w sections, positions up to 2e4 (DM times)."""
    E.config(False, False)
    half = d // 2
    a, b = sorted(min(c, half) for c in cut)
    secs = (a, b - a, half - b)
    r = np.random.default_rng(seed)
    try:
        x = r.standard_normal((n, h, d)).astype(np.float32)
        x = val(bits_of(x)) if bf16 else x
        pos = np.floor(r.uniform(0, pmax, (n, 3))).astype(np.float32)
        X = E.empty((n, h + pad, d), np.uint16 if bf16 else np.float32)
        X[:, :h] = bits_of(x) if bf16 else x
        view = X[:, :h]
        el = _el(view)
        st_ = E.call("mrope_apply", emu_lib.ptr(view), BF16 if bf16 else FP32, n, h, d, el[0], el[1],
                     emu_lib.ptr(E.array(pos)), *secs, ctypes.c_float(theta), None)
        assert st_ == 0
        want = omrope.apply(x, pos, secs, float(np.float32(theta)))
        assert_parity(val(X[:, :h]) if bf16 else X[:, :h], want, "bf16" if bf16 else "fp32", "mrope")
        assert (X[:, h:] == 0).all()
    finally:
        E.free_all()


@settings(max_examples=20, **SETTINGS)
@given(n=st.integers(1, 5000), bf16=st.booleans(), guided=st.booleans(), mirror=st.booleans(),
       w=st.sampled_from([0.0, 1.0, 3.0, 7.5]), sig=st.tuples(st.floats(0, 1), st.floats(0, 1)),
       seed=st.integers(0, 10 ** 6))
def test_euler_random_problems(E, n, bf16, guided, mirror, w, sig, seed):
    E.config(False, False)
    s0, s1 = float(np.float32(max(sig))), float(np.float32(min(sig)))
    r = np.random.default_rng(seed)
    try:
        x0 = r.standard_normal(n).astype(np.float32)
        vc = r.standard_normal(n).astype(np.float32)
        vb = r.standard_normal(n).astype(np.float32)
        if bf16:
            vc, vb = val(bits_of(vc)), val(bits_of(vb))
        code = BF16 if bf16 else FP32
        X = E.array(x0)
        XB = E.empty((n,), np.uint16) if mirror else None
        VC = E.array(bits_of(vc) if bf16 else vc)
        VB = E.array(bits_of(vb) if bf16 else vb)
        if guided:
            st_ = E.call("flow_cfg_euler_step", emu_lib.ptr(X), emu_lib.ptr(VC), emu_lib.ptr(VB), code, n,
                         ctypes.c_float(w), ctypes.c_float(s0), ctypes.c_float(s1), emu_lib.ptr(XB), None)
            want = ocfg.euler_step(x0, vc, vb, w, s0, s1)
        else:
            st_ = E.call("flow_euler_step", emu_lib.ptr(X), emu_lib.ptr(VC), code, n, ctypes.c_float(s0),
                         ctypes.c_float(s1), emu_lib.ptr(XB), None)
            want = oeuler.step(x0, vc, s0, s1)
        assert st_ == 0
        assert_parity(X, want, "fp32", "euler")
        if mirror:
            np.testing.assert_array_equal(XB, W.bf16_bits(np.array(X)))
    finally:
        E.free_all()
