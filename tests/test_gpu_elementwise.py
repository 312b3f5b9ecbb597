"""GPU parity of the bandwidth kernels: flow_euler_step and mrope_apply,
against the fp64 oracle on the same seeded input bytes."""
import numpy as np
import pytest

import workloads as W
from oracle import euler as oeuler
from oracle import layout as olayout
from oracle import mrope as omrope
from tests.gpu_util import assert_parity, device, say, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _mot():
    import multimodal_diffusion_transformer_amd as mot
    return mot


@pytest.mark.parametrize("n", [1, 7, 8, 4099, 4_423_681])
@pytest.mark.parametrize("vdt", ["bf16", "fp32"])
def test_euler_parity(n, vdt):
    dev = device()
    mot = _mot()
    say("euler n=%d v=%s" % (n, vdt))
    x0 = W.make(10, 1, (n,), "fp32").f32
    vt = W.make(10, 2, (n,), vdt)
    x = torch.from_numpy(x0.copy()).to(dev)
    v = W.to_torch(vt, dev)
    mot.flow_euler_step(x, v, 1.0, 0.75)
    torch.cuda.synchronize()
    want = oeuler.step(x0, vt.f32, 1.0, 0.75)
    assert_parity(to_np(x), want, "fp32", "euler")
    assert np.abs(to_np(x) - want).max() <= 1e-6


def test_euler_zero_velocity_is_bitwise_identity_and_mirror_is_rne():
    dev = device()
    mot = _mot()
    n = 1_000_003
    x0 = W.make(11, 1, (n,), "fp32").f32
    x = torch.from_numpy(x0.copy()).to(dev)
    v = torch.zeros(n, dtype=torch.bfloat16, device=dev)
    xb = torch.empty(n, dtype=torch.bfloat16, device=dev)
    mot.flow_euler_step(x, v, 0.6, 0.2, x_bf16=xb)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(x).view(np.uint32), x0.view(np.uint32))
    np.testing.assert_array_equal(xb.cpu().view(torch.int16).numpy().view(np.uint16),
                                  W.bf16_bits(x0))


def test_euler_recovers_x0_on_the_rectified_flow_path():
    dev = device()
    mot = _mot()
    n = 65536
    eps = W.make(12, 1, (n,), "fp32").f32
    x0 = W.make(12, 2, (n,), "fp32").f32
    vstar = (eps.astype(np.float64) - x0).astype(np.float32)
    x = torch.from_numpy(eps.copy()).to(dev)
    v = torch.from_numpy(vstar).to(dev)
    sched = oeuler.linear_schedule(10)
    for s, sn in zip(sched[:-1], sched[1:]):
        mot.flow_euler_step(x, v, s, sn)
    torch.cuda.synchronize()
    assert np.abs(to_np(x) - x0).max() < 1e-5


def _rope_case(wl):
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h, d = len(reg), wl.n_heads, wl.head_dim
    y = W.make(wl.wid, 40, (n, 3, h, d), wl.dtype)
    return pos, y


@pytest.mark.parametrize("name", ["tiny_fp32", "policy_bf16", "stream_chunk_bf16"])
def test_mrope_parity_strided_qk_views(name):
    dev = device()
    mot = _mot()
    wl = W.BY_NAME[name]
    say("mrope %s" % name)
    pos, y = _rope_case(wl)
    Y = W.to_torch(y, dev).contiguous()
    P = torch.from_numpy(pos).to(dev)
    mot.mrope_apply(Y[:, 0], P, wl.sections, wl.theta)
    mot.mrope_apply(Y[:, 1], P, wl.sections, wl.theta)
    torch.cuda.synchronize()
    got = to_np(Y)
    for part in (0, 1):
        want = omrope.apply(y.f32[:, part], pos, wl.sections, wl.theta)
        assert_parity(got[:, part], want, wl.dtype, "mrope part %d" % part)
    # V untouched
    np.testing.assert_array_equal(got[:, 2], y.f32[:, 2])


def test_mrope_text_positions_zero_is_identity():
    dev = device()
    mot = _mot()
    x = W.make(13, 1, (64, 8, 128), "bf16")
    X = W.to_torch(x, dev)
    P = torch.zeros((64, 3), dtype=torch.float32, device=dev)
    mot.mrope_apply(X, P, (16, 24, 24), 1e4)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(X), x.f32)
