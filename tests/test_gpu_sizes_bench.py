"""GPU parity at the sizes and launch shapes the benchmark times: the 480p
text-to-video step (25,474 tokens, 24 heads of 128, hidden 3,072).

* The Euler update over all 24,960 x 3,072 noisy-latent elements (plus a
  ragged tail) with the bf16 mirror.  The kernel's grid is capped at 4,096
  workgroups, so at this size each lane makes several trips of its
  grid-stride loop, which the smaller cases never do.
* mRoPE of K as the strided view of the packed [N, 3, H, D] QKV buffer,
  checked on sampled tokens (all AR tokens, the AR/DM boundary, random DM
  tokens, the last token): the oracle rotates each token on its own.
* The attention launch of the benchmark: Q, K and V strided views of that
  buffer, Q rotated on load from the token positions (the kernel instance
  the benchmark times), no LSE, checked on sampled rows and heads.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention as oattn
from oracle import euler as oeuler
from oracle import layout as olayout
from oracle import mrope as omrope
from tests.gpu_util import assert_parity, device, say, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

WORKLOAD = "t2v480p_bf16"


def _mot():
    import multimodal_diffusion_transformer_amd as mot
    return mot


def test_euler_bench_size_with_mirror():
    dev = device()
    mot = _mot()
    wl = W.BY_NAME[WORKLOAD]
    _, _, n_noisy = W.region_counts(wl.segments)
    n = n_noisy * wl.hidden + 3
    sigma, sigma_next = wl.sigmas[0], wl.sigmas[1]
    say("euler 480p n=%d sigma %g -> %g" % (n, sigma, sigma_next))
    x0 = W.make(20, 1, (n,), "fp32").f32
    vt = W.make(20, 2, (n,), "bf16")
    x = torch.tensor(x0, device=dev)  # a copy: x0 stays the oracle's input
    v = W.to_torch(vt, dev)
    xb = torch.empty(n, dtype=torch.bfloat16, device=dev)
    mot.flow_euler_step(x, v, sigma, sigma_next, x_bf16=xb)
    torch.cuda.synchronize()
    got = to_np(x)
    want = oeuler.step(x0, vt.f32, sigma, sigma_next)
    assert_parity(got, want, "fp32", "euler 480p")
    # one fused multiply-add per element: within half an ulp of |x| < 8
    assert np.abs(got - want).max() <= 1e-6
    # the mirror is the round-to-nearest-even bf16 of the updated value, bit for bit
    np.testing.assert_array_equal(xb.cpu().view(torch.int16).numpy().view(np.uint16),
                                  W.bf16_bits(got))


def sampled_tokens(n, n_ar, seed, n_random):
    """All AR tokens, 64 on each side of the AR/DM boundary, n_random DM
    tokens and the last token, sorted."""
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([
        np.arange(n_ar), np.arange(n_ar - 64, n_ar + 64),
        rng.choice(np.arange(n_ar, n), size=n_random, replace=False), [n - 1]]))


def test_mrope_bench_size_k_view_sampled_tokens():
    dev = device()
    mot = _mot()
    wl = W.BY_NAME[WORKLOAD]
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h, d = len(reg), wl.n_heads, wl.head_dim
    say("mrope 480p K view n=%d h=%d d=%d" % (n, h, d))
    k = W.make(21, 1, (n, h, d), "bf16")
    Y = torch.empty((n, 3, h, d), dtype=torch.bfloat16, device=dev)
    Y[:, 1] = W.to_torch(k, dev)
    Y[:, 0].fill_(1.0)   # Q and V slots: sentinels that must stay untouched
    Y[:, 2].fill_(-2.0)
    P = torch.from_numpy(pos).to(dev)
    mot.mrope_apply(Y[:, 1], P, wl.sections, wl.theta)
    torch.cuda.synchronize()
    rows = sampled_tokens(n, n_ar, 21, 2048)
    got = to_np(Y.index_select(0, torch.from_numpy(rows).to(dev)))
    want = omrope.apply(k.f32[rows], pos[rows], wl.sections, wl.theta)
    assert_parity(got[:, 1], want, "bf16", "mrope 480p K")
    assert (got[:, 0] == 1.0).all() and (got[:, 2] == -2.0).all()


ATTN_HEADS = [0, 11, 23]


def test_attention_bench_launch_sampled_rows():
    dev = device()
    mot = _mot()
    wl = W.BY_NAME[WORKLOAD]
    pos, reg, n_ar = olayout.build(wl.segments)
    n, h, d = len(reg), wl.n_heads, wl.head_dim
    say("attention 480p bench launch n=%d (Q rotated on load, strided Q/K/V)" % n)
    q = W.make(22, W.T_Q, (n, h, d), "bf16")
    k = W.make(22, W.T_K, (n, h, d), "bf16")   # taken as already rotated
    v = W.make(22, W.T_V, (n, h, d), "bf16")
    Y = torch.empty((n, 3, h, d), dtype=torch.bfloat16, device=dev)
    for part, t in enumerate((q, k, v)):
        Y[:, part] = W.to_torch(t, dev)
    P = torch.from_numpy(pos).to(dev)
    O = torch.empty((n, h * d), dtype=torch.bfloat16, device=dev)
    mot.mot_attention_fwd(Y[:, 0], Y[:, 1], Y[:, 2], O.view(n, h, d), mask=W.AR_CAUSAL_DM_FULL,
                          n_ar=n_ar, q_pos=P, sections=wl.sections, theta=wl.theta)
    torch.cuda.synchronize()
    rows = sampled_tokens(n, n_ar, 22, 64)
    got = to_np(O.view(n, h, d).index_select(0, torch.from_numpy(rows).to(dev)))[:, ATTN_HEADS]
    qr = omrope.apply(q.f32[rows], pos[rows], wl.sections, wl.theta)
    want = oattn.attention_rows(qr, k.f32, v.f32, rows, ATTN_HEADS, 0, W.AR_CAUSAL_DM_FULL,
                                n_ar=n_ar)
    assert_parity(got, want, "bf16", "attention 480p bench launch")
