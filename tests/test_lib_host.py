"""CPU tests of the C-ABI library: it loads, exports what the header
declares, and its host-side logic (layout, tile classifier, argument checks)
matches the oracle exactly.  No device work is launched here."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import json
from fractions import Fraction

import workloads as W
from oracle import layout as olayout
from oracle import mask as omask
from oracle import schedule as oschedule

mot = pytest.importorskip("multimodal_diffusion_transformer_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "motattn.h")


def _declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:mot_status|int|const char\*)\s+(\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary_calls():
    names = _declared_functions()
    for n in ("mot_qkv_project", "mrope_apply", "mot_attention_fwd", "flow_euler_step"):
        assert n in names
    assert sorted(names) == sorted(mot.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mot.LIB_PATH)
    for n in _declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", mot.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(_declared_functions()) <= exported


def test_abi_version_and_status_strings():
    assert mot.mot_abi_version() == 2
    assert mot.mot_status_string(0) == "ok"
    assert "invalid" in mot.mot_status_string(1)


@pytest.mark.parametrize("wl", W.WORKLOADS, ids=lambda w: w.name)
def test_layout_bitwise_equals_oracle(wl):
    p1, r1, a1 = mot.mot_build_layout(wl.segments)
    p2, r2, a2 = olayout.build(wl.segments)
    assert a1 == a2
    np.testing.assert_array_equal(r1, r2)
    np.testing.assert_array_equal(p1.view(np.uint32), p2.view(np.uint32))


def test_layout_bitwise_on_mixed_rates():
    segs = [W.text(5), *W.eos_bog(), W.video(W.DM_CLEAN, 2, 2, 3, 4, fps=30.0),
            W.audio(W.DM_CLEAN, 17), W.action(W.DM_CLEAN, 9, hz=15.0),
            W.video(W.DM_NOISY, 3, 2, 3, 4, fps=30.0), W.audio(W.DM_NOISY, 33, step0=17),
            W.action(W.DM_NOISY, 21, hz=10.0, step0=9), W.proprio(W.DM_NOISY, 2)]
    p1, r1, a1 = mot.mot_build_layout(segs)
    p2, r2, a2 = olayout.build(segs)
    np.testing.assert_array_equal(p1.view(np.uint32), p2.view(np.uint32))
    np.testing.assert_array_equal(r1, r2)


@pytest.mark.parametrize("segs", [
    [W.text(3), W.video(W.DM_NOISY, 1, 1, 2, 2), W.video(W.DM_CLEAN, 1, 1, 2, 2)],
    [W.text(3), W.action(W.DM_NOISY, 2), W.video(W.DM_NOISY, 1, 1, 2, 2)],
    [W.text(3), W.video(W.DM_NOISY, 1, 1, 2, 2), W.text(2)],
    [W.text(0)],
])
def test_layout_rejects_bad_order(segs):
    with pytest.raises(mot.MotError):
        mot.mot_build_layout(segs)


def test_layout_rejects_counts_past_int64():
    def status(segs):
        arr = (mot.mot_segment * len(segs))(*segs)
        n, n_ar = ctypes.c_int64(0), ctypes.c_int64(0)
        return mot.raw_call("mot_build_layout", arr, len(segs), 0, ctypes.byref(n),
                            ctypes.byref(n_ar), None, None), n.value

    text = mot.mot_segment(W.AR, W.TEXT, 4, 0, 1, 0, 0, 0.0, -1, 0)
    big_video = mot.mot_segment(W.DM_NOISY, W.VIDEO, 0, 1 << 40, 1 << 20, 1 << 10, 1 << 10, 24.0, -1, 0)
    assert status([text, big_video]) == (mot.MOT_ERR_INVALID_ARG, 0)
    half = mot.mot_segment(W.AR, W.TEXT, 1 << 62, 0, 1, 0, 0, 0.0, -1, 0)
    assert status([half, half, half, half]) == (mot.MOT_ERR_INVALID_ARG, 0)
    late = mot.mot_segment(W.DM_NOISY, W.VIDEO, 0, 2, 1, 4, 4, 24.0, (1 << 63) - 1, 0)
    assert status([text, late]) == (mot.MOT_ERR_INVALID_ARG, 0)
    far = mot.mot_segment(W.DM_NOISY, W.ACTION, 8, 0, 1, 0, 0, 15.0, -1, (1 << 63) - 4)
    assert status([text, far]) == (mot.MOT_ERR_INVALID_ARG, 0)
    # the largest counts that fit are sized, not rejected
    ok = mot.mot_segment(W.DM_NOISY, W.VIDEO, 0, 1 << 20, 1 << 20, 1 << 10, 1 << 10, 24.0, -1, 0)
    assert status([text, ok]) == (mot.MOT_ERR_INVALID_ARG, 4 + (1 << 60))


@pytest.mark.parametrize("case", [
    dict(nq=25474, nk=25474, q0=0, mask=W.AR_CAUSAL_DM_FULL, n_ar=514),
    dict(nq=2451, nk=2451, q0=0, mask=W.AR_CAUSAL_DM_FULL, n_ar=258),
    dict(nq=300, nk=700, q0=400, mask=W.AR_CAUSAL_DM_FULL, n_ar=513),
    dict(nq=1440, nk=13218, q0=11778, mask=W.CHUNK_CAUSAL_KV, n_prefix=258, chunk_len=1440),
    dict(nq=3 * 37 + 5, nk=258 + 3 * 37 + 5, q0=258, mask=W.CHUNK_CAUSAL_KV, n_prefix=258, chunk_len=37),
])
@pytest.mark.parametrize("bm,bn", [(128, 64), (128, 128), (32, 64)])
def test_host_tile_classes_equal_oracle(case, bm, bn):
    a = mot.mask_args(**case)
    got = mot.mot_tile_classes_host(a, bm, bn)
    m = omask.materialize(case["nq"], case["nk"], case["q0"], case["mask"],
                          case.get("n_ar", 0), case.get("n_prefix", 0), case.get("chunk_len", 1))
    want = omask.tile_classes(m, bm, bn)
    np.testing.assert_array_equal(got, want)


def test_tile_counts_t2v480p_at_128():
    a = mot.mask_args(25474, 25474, 0, W.AR_CAUSAL_DM_FULL, n_ar=514)
    tc = mot.mot_tile_classes_host(a, 128, 128)
    assert tc.size == 200 * 200
    assert int((tc == omask.EMPTY).sum()) == 790 and int((tc == omask.PARTIAL).sum()) == 200


# ---- flow-shifted noise schedule (host only) ----
_SETTINGS = json.load(open(os.path.join(ROOT, "tests", "golden", "recommended_sampler_settings.json"),
                           encoding="utf-8"))["settings"]
_SCHED = sorted({(r["steps"], float(r["shift"])) for r in _SETTINGS}
                | {(n, s) for n in (1, 2, 3, 5, 8, 13, 64) for s in (0.3, 1.0, 2.5, 3.0, 7.0, 12.5)})


def _nearest_f32(x: Fraction) -> np.float32:
    """The float32 nearest to the rational x (ties to even), by comparing
    the candidates around the double nearest to x exactly."""
    f = np.float32(float(x))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    def key(c):
        bits = int(np.array(c, dtype=np.float32).view(np.uint32))
        return (abs(Fraction(float(c)) - x), bits & 1)
    return min(cands, key=key)


@pytest.mark.parametrize("case", _SCHED, ids=lambda c: "n%d_s%g" % c)
def test_sigma_schedule_bitwise_equals_oracle(case):
    n, shift = case
    got = mot.mot_sigma_schedule(n, shift)
    want = np.array(oschedule.shifted_schedule(n, shift), dtype=np.float64).astype(np.float32)
    assert got.dtype == np.float32 and got.shape == (n + 1,)
    assert got.tobytes() == want.tobytes()
    assert got[0] == 1.0 and got[-1] == 0.0


@pytest.mark.parametrize("case", [c for c in _SCHED if c[0] <= 13], ids=lambda c: "n%d_s%g" % c)
def test_sigma_schedule_is_the_nearest_float_of_the_exact_value(case):
    n, shift = case
    got = mot.mot_sigma_schedule(n, shift)
    s = Fraction(shift)
    for k in range(n + 1):
        exact = s * (n - k) / (n + (s - 1) * (n - k))
        assert got[k] == _nearest_f32(exact), (k, float(exact))


def test_sigma_schedule_rejects_bad_args():
    buf = np.zeros(8, dtype=np.float32)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    for n, shift, ptr in [(0, 5.0, p), (-3, 5.0, p), (4, 0.0, p), (4, -2.0, p),
                          (4, float("inf"), p), (4, float("nan"), p), (4, 5.0, None),
                          (4, 2.0 ** -21, p), (4, 1e-300, p), (4, 2.0 ** 21, p)]:
        assert mot.raw_call("mot_sigma_schedule", n, ctypes.c_double(shift), ptr) == \
            mot.MOT_ERR_INVALID_ARG
    assert not buf.any()


# ---- argument checks: every one returns before any launch ----
def _args(**kw):
    a = mot.mot_attn_args()
    a.q = a.k = a.v = a.o = 4096
    a.dt, a.n_heads, a.head_dim, a.mask = mot.MOT_BF16, 2, 128, mot.MOT_AR_CAUSAL_DM_FULL
    a.nq = a.nk = 64
    a.q_ts = a.k_ts = a.v_ts = a.o_ts = 256
    a.q_hs = a.k_hs = a.v_hs = a.o_hs = 128
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(head_dim=96), dict(n_heads=0), dict(nq=-1), dict(nk=10), dict(nq=0, nk=-1),
    dict(nq=0, head_dim=96),
    dict(q_ts=7), dict(o_hs=0), dict(q=4100), dict(dt=5), dict(mask=7),
    dict(mask=mot.MOT_CHUNK_CAUSAL_KV, chunk_len=0),
    dict(mask=mot.MOT_CHUNK_CAUSAL_KV, chunk_len=8, n_prefix=10, q0=5, nk=100),
    dict(q_pos=4096, sec_t=1, sec_h=1, sec_w=1),
    dict(scale=-1.0),
    # grouped heads: H_kv must divide H; the batch: count and strides
    dict(n_kv_heads=3), dict(n_kv_heads=-1), dict(n_batch=-1), dict(n_batch=65536),
    dict(n_batch=2, k_bs=-8), dict(n_batch=2, q_bs=4), dict(n_batch=2, o_bs=12),
])
def test_attention_rejects_bad_args(kw):
    st = mot.raw_call("mot_attention_fwd", ctypes.byref(_args(**kw)), None)
    assert st == mot.MOT_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    # bf16 rotates Q on load only; K is rotated beforehand
    dict(k_pos=4096, sec_t=16, sec_h=24, sec_w=24, theta=1e4),
    # a 64-row K tile past 4 GiB, and key counts past 32 bits
    dict(k_ts=1 << 25, k_hs=128),
    dict(nk=1 << 31),
])
def test_attention_bf16_unsupported(kw):
    st = mot.raw_call("mot_attention_fwd", ctypes.byref(_args(**kw)), None)
    assert st == mot.MOT_ERR_UNSUPPORTED


@pytest.mark.parametrize("dt", [mot.MOT_BF16, mot.MOT_FP32])
def test_attention_with_no_query_rows_is_a_no_op(dt):
    # the pointers are never dereferenced: nothing is launched
    for kw in (dict(nq=0), dict(nq=0, nk=0), dict(nq=0, mask=mot.MOT_CHUNK_CAUSAL_KV, chunk_len=0),
               dict(nq=0, q=None, o=None)):
        assert mot.raw_call("mot_attention_fwd", ctypes.byref(_args(dt=dt, **kw)), None) == mot.MOT_OK


def test_launches_past_one_dispatch_are_unsupported():
    # Sizes whose grid would exceed 2^32 - 1 work-items: every call returns
    # UNSUPPORTED before any launch (the pointers are never dereferenced).
    vp = ctypes.c_void_p
    # bf16 attention: chunk mode lets nq exceed nk; 2 * 4 heads * (2^30 + 512) > 2^32
    a = _args(mask=mot.MOT_CHUNK_CAUSAL_KV, chunk_len=64, nq=1 << 30, nk=64, n_heads=4)
    assert mot.raw_call("mot_attention_fwd", ctypes.byref(a), None) == mot.MOT_ERR_UNSUPPORTED
    a = _args(mask=mot.MOT_CHUNK_CAUSAL_KV, chunk_len=64, nq=1 << 32, nk=64, n_heads=1,
              dt=mot.MOT_FP32)
    assert mot.raw_call("mot_attention_fwd", ctypes.byref(a), None) == mot.MOT_ERR_UNSUPPORTED
    # mRoPE: 2^29 tokens x 16 lanes
    assert mot.raw_call("mrope_apply", vp(4096), 0, 1 << 29, 1, 128, 1024, 128, vp(4096), 16, 24,
                        24, ctypes.c_float(1e4), None) == mot.MOT_ERR_UNSUPPORTED
    # mRoPE at D = 80: 25 tokens per 256-lane workgroup, at most 2^24 - 1 workgroups
    assert mot.raw_call("mrope_apply", vp(4096), 0, 25 * ((1 << 24) - 1) + 1, 1, 80, 1024, 80, vp(4096), 10,
                        15, 15, ctypes.c_float(1e4), None) == mot.MOT_ERR_UNSUPPORTED
    # projection: 2^31 rows x 2^16 columns of 128 x 128 tiles; fp32 d_out = 2^28
    assert mot.raw_call("mot_qkv_project", vp(4096), vp(4096), vp(4096), vp(4096), 1 << 31, 0, 64,
                        1 << 16, 0, 0, None) == mot.MOT_ERR_UNSUPPORTED
    assert mot.raw_call("mot_qkv_project", vp(4096), vp(4096), vp(4096), vp(4096), 16, 0, 4,
                        1 << 28, 1, 1, None) == mot.MOT_ERR_UNSUPPORTED
    # mask of the long 480p sequence: 76,954^2 entries > 2^32
    m = mot.mask_args(76954, 76954, 0, W.AR_CAUSAL_DM_FULL, n_ar=514)
    assert mot.raw_call("mot_mask_materialize", ctypes.byref(m), vp(4096), 128, 64, None,
                        None) == mot.MOT_ERR_UNSUPPORTED
    # tile classes at 1 x 1 tiles of the same sequence
    assert mot.raw_call("mot_mask_materialize", ctypes.byref(m), None, 1, 1, vp(4096),
                        None) == mot.MOT_ERR_UNSUPPORTED
    # q0 + nq past int64 is rejected, not wrapped
    m = mot.mask_args(1 << 62, 64, (1 << 63) - 2, W.AR_CAUSAL_DM_FULL)
    assert mot.raw_call("mot_mask_materialize", ctypes.byref(m), vp(4096), 128, 64, None,
                        None) == mot.MOT_ERR_INVALID_ARG


def test_projection_and_rope_and_euler_reject_bad_args():
    vp = ctypes.c_void_p
    # projection: n_ar > n_rows; unaligned; bf16 with d_in not a multiple of 64
    assert mot.raw_call("mot_qkv_project", vp(4096), vp(4096), vp(4096), vp(4096), 10, 11, 64,
                        64, 0, 0, None) == mot.MOT_ERR_INVALID_ARG
    assert mot.raw_call("mot_qkv_project", vp(4098), vp(4096), vp(4096), vp(4096), 10, 5, 64,
                        64, 0, 0, None) == mot.MOT_ERR_INVALID_ARG
    assert mot.raw_call("mot_qkv_project", vp(4096), vp(4096), vp(4096), vp(4096), 10, 5, 96,
                        64, 0, 0, None) == mot.MOT_ERR_UNSUPPORTED
    # rope: sections that do not cover D/2; head_dim 96
    assert mot.raw_call("mrope_apply", vp(4096), 0, 10, 2, 128, 256, 128, vp(4096), 16, 24, 23,
                        ctypes.c_float(1e4), None) == mot.MOT_ERR_INVALID_ARG
    assert mot.raw_call("mrope_apply", vp(4096), 0, 10, 2, 96, 256, 128, vp(4096), 16, 16, 16,
                        ctypes.c_float(1e4), None) == mot.MOT_ERR_INVALID_ARG
    # euler: negative n; unaligned v; zero n is a no-op
    assert mot.raw_call("flow_euler_step", vp(4096), vp(4096), 0, -1, ctypes.c_float(1.0),
                        ctypes.c_float(0.5), None, None) == mot.MOT_ERR_INVALID_ARG
    assert mot.raw_call("flow_euler_step", vp(4096), vp(4098), 0, 64, ctypes.c_float(1.0),
                        ctypes.c_float(0.5), None, None) == mot.MOT_ERR_INVALID_ARG
    assert mot.raw_call("flow_euler_step", None, None, 0, 0, ctypes.c_float(1.0),
                        ctypes.c_float(0.5), None, None) == mot.MOT_OK
    # empty projection and rope are no-ops that touch nothing (null pointers allowed)
    assert mot.raw_call("mot_qkv_project", None, None, None, None, 0, 0, 64, 64, 0, 0,
                        None) == mot.MOT_OK
    assert mot.raw_call("mrope_apply", None, 0, 0, 2, 128, 256, 128, None, 16, 24, 24,
                        ctypes.c_float(1e4), None) == mot.MOT_OK
    # guided euler: a missing or unaligned velocity, a bad dtype, a guidance
    # that is not finite; zero n is a no-op
    f = ctypes.c_float
    for args in [(vp(4096), vp(4096), None, 0, 64, f(3.0)), (vp(4096), vp(4096), vp(4100), 0, 64, f(3.0)),
                 (vp(4096), vp(4096), vp(4096), 7, 64, f(3.0)),
                 (vp(4096), vp(4096), vp(4096), 0, 64, f(float("inf"))),
                 (vp(4096), vp(4096), vp(4096), 0, 64, f(float("nan"))),
                 (vp(4096), vp(4096), vp(4096), 0, -1, f(3.0))]:
        assert mot.raw_call("flow_cfg_euler_step", *args, f(1.0), f(0.5), None,
                            None) == mot.MOT_ERR_INVALID_ARG, args
    assert mot.raw_call("flow_cfg_euler_step", None, None, None, 0, 0, f(3.0), f(1.0), f(0.5), None,
                        None) == mot.MOT_OK
    # region linear: unknown epilogue, residual missing for ADD or given
    # otherwise, misaligned residual; empty is a no-op
    P = vp(4096)
    for epi, res in [(3, None), (-1, None), (mot.MOT_EPI_ADD, None), (mot.MOT_EPI_GELU, P),
                     (mot.MOT_EPI_NONE, P), (mot.MOT_EPI_ADD, vp(4100))]:
        assert mot.raw_call("mot_region_linear", P, P, P, P, 10, 5, 64, 64, 0, 0, epi, res,
                            None) == mot.MOT_ERR_INVALID_ARG, (epi, res)
    assert mot.raw_call("mot_region_linear", None, None, None, None, 0, 0, 64, 64, 0, 0,
                        mot.MOT_EPI_GELU, None, None) == mot.MOT_OK
    # layernorm: hidden not a multiple of 8, eps not positive, a room with
    # rows but no parameters, misaligned, too wide; empty is a no-op
    for args in [(10, 4, 100, P, P, P, P, f(1e-6)), (10, 4, 64, P, P, P, P, f(0.0)),
                 (10, 4, 64, P, P, P, P, f(float("nan"))), (10, 4, 64, None, P, P, P, f(1e-6)),
                 (10, 4, 64, P, P, None, None, f(1e-6)), (10, 4, 64, P, vp(4100), P, P, f(1e-6))]:
        assert mot.raw_call("mot_layernorm_region", P, P, *args, 0, 0, None) == \
            mot.MOT_ERR_INVALID_ARG, args
    assert mot.raw_call("mot_layernorm_region", P, P, 10, 4, 8200, P, P, P, P, f(1e-6), 0, 0,
                        None) == mot.MOT_ERR_UNSUPPORTED
    assert mot.raw_call("mot_layernorm_region", None, None, 0, 0, 64, None, None, None, None,
                        f(1e-6), 0, 0, None) == mot.MOT_OK
    # attention merge: part count, head_dim, strides, alignment, dtype; nq 0 is a no-op
    for args in [(P, P, 0, 0, 10, 2, 128, 256, 128, P, 256, 128, None, 0),
                 (P, P, 17, 0, 10, 2, 128, 256, 128, P, 256, 128, None, 0),
                 (P, P, 2, 0, 10, 2, 96, 256, 128, P, 256, 128, None, 0),
                 (P, P, 2, 4, 10, 2, 128, 256, 128, P, 256, 128, None, 0),
                 (P, P, 2, 0, 10, 2, 128, 250, 128, P, 256, 128, None, 0),
                 (vp(4100), P, 2, 0, 10, 2, 128, 256, 128, P, 256, 128, None, 0),
                 (P, vp(4098), 2, 0, 10, 2, 128, 256, 128, P, 256, 128, None, 0),
                 (P, P, 2, 0, 10, 2, 128, 256, 128, P, 256, 128, None, 5),
                 (None, P, 2, 0, 10, 2, 128, 256, 128, P, 256, 128, None, 0)]:
        assert mot.raw_call("mot_attention_merge", *args, None) == mot.MOT_ERR_INVALID_ARG, args
    assert mot.raw_call("mot_attention_merge", None, None, 2, 0, 0, 2, 128, 256, 128, None, 256, 128,
                        None, 0, None) == mot.MOT_OK
    assert mot.raw_call("mot_attention_merge", P, P, 2, 0, 1 << 40, 2, 128, 256, 128, P, 256, 128,
                        None, 0, None) == mot.MOT_ERR_UNSUPPORTED
