"""GPU parity of the key-split attention: mot_attention_merge on its own,
and the streaming call with its keys split over a batch of two launches and
merged through their LSE (pipeline.StreamState(split=2)), against the
oracle (oracle.attention.merge, oracle.streaming.RollingCache)."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as oattn
from oracle import layout as olayout
from oracle import streaming as ostream
from tests.gpu_util import BF16_LSE_ATOL, assert_parity, device, say, stream_workload, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _mot():
    import multimodal_diffusion_transformer_amd as mot
    return mot


@pytest.mark.parametrize("dtype,d,parts", [("bf16", 128, 2), ("bf16", 64, 3), ("fp32", 128, 2), ("fp32", 64, 1),
                                           ("bf16", 80, 3)])
def test_merge_parity(dtype, d, parts):
    dev = device()
    mot = _mot()
    nq, h = 333, 3
    say("merge %s d=%d parts=%d" % (dtype, d, parts))
    o = W.make(60, 1, (parts, nq, h, d), dtype)
    l = W.make(60, 2, (parts, h, nq), "fp32")
    lse_np = l.f32 * 3.0  # spread the weights
    O = torch.empty((nq, h, d), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device=dev)
    L = torch.empty((h, nq), dtype=torch.float32, device=dev)
    mot.mot_attention_merge(W.to_torch(o, dev), torch.tensor(lse_np, device=dev), O, lse=L)
    torch.cuda.synchronize()
    want, want_l = oattn.merge(o.f32, lse_np)
    assert_parity(to_np(O), want, dtype, "merge")
    np.testing.assert_allclose(to_np(L), want_l, atol=1e-5, rtol=0)


def test_key_split_launch_equals_attention_over_all_keys():
    """Full attention of 300 queries over 1,030 keys, the keys split in two
    halves over a batch of two launches and merged."""
    dev = device()
    mot = _mot()
    nq, nk, h, d = 300, 1030, 4, 128
    half = nk // 2
    q = W.make(61, 1, (nq, h, d), "bf16")
    k = W.make(61, 2, (nk, h, d), "bf16")
    v = W.make(61, 3, (nk, h, d), "bf16")
    Q, K, V = (W.to_torch(t, dev) for t in (q, k, v))
    K2 = torch.as_strided(K, (2, half, h, d), (half * K.stride(0),) + tuple(K.stride()))
    V2 = torch.as_strided(V, (2, half, h, d), (half * V.stride(0),) + tuple(V.stride()))
    Op = torch.empty((2, nq, h, d), dtype=torch.bfloat16, device=dev)
    Lp = torch.empty((2, h, nq), dtype=torch.float32, device=dev)
    mot.mot_attention_fwd(Q.unsqueeze(0).expand(2, nq, h, d), K2, V2, Op, mask=W.AR_CAUSAL_DM_FULL, q0=0,
                          n_ar=0, lse=Lp)
    O = torch.empty((nq, h, d), dtype=torch.bfloat16, device=dev)
    L = torch.empty((h, nq), dtype=torch.float32, device=dev)
    mot.mot_attention_merge(Op, Lp, O, lse=L)
    torch.cuda.synchronize()
    want, lse = oattn.attention(q.f32, k.f32, v.f32, nk, W.AR_CAUSAL_DM_FULL, n_ar=0)
    assert_parity(to_np(O), want, "bf16", "split + merge")
    np.testing.assert_allclose(to_np(L), lse, atol=BF16_LSE_ATOL, rtol=0)


@pytest.mark.parametrize("size", ["stream_chunk_bf16", "mini"])
def test_streaming_rollout_with_split_keys(size):
    """The streaming workload with each call's keys split in two and merged:
    two chunks x 4 steps against the oracle's rolling cache (at the reduced
    size: every chunk, through the ring wrap)."""
    dev = device()
    from multimodal_diffusion_transformer_amd import pipeline as P
    wl = stream_workload(size)
    h, d = wl.n_heads, wl.head_dim
    ft = wl.stream_views * wl.stream_gh * wl.stream_gw
    slots = wl.stream_history_frames
    n_prefix = wl.stream_text + 2
    pos, reg, n_ar = olayout.build(wl.segments)
    pre_k = W.make(3, 50, (n_prefix + slots * ft, h, d), "bf16")
    pre_v = W.make(3, 51, (n_prefix + slots * ft, h, d), "bf16")
    st = P.StreamState(h, d, n_prefix, ft, slots, wl.sections, wl.theta, device=dev, split=2)
    st.fill(W.to_torch(pre_k, dev), W.to_torch(pre_v, dev), torch.from_numpy(pos[:n_prefix + slots * ft]).to(dev))
    oc = ostream.RollingCache(pre_k.f32[:n_prefix], pre_v.f32[:n_prefix], pos[:n_prefix],
                              pre_k.f32[n_prefix:], pre_v.f32[n_prefix:],
                              pos[n_prefix:n_prefix + slots * ft], ft, wl.sections, wl.theta)
    t0 = n_ar + 15000.0
    chunk_pos = pos[n_prefix + slots * ft:].copy()
    O = torch.empty((ft, h, d), dtype=torch.bfloat16, device=dev)
    rng = np.random.default_rng(62)
    for c in range(2 if size == "stream_chunk_bf16" else wl.stream_chunks):
        cp = chunk_pos.copy()
        cp[:, 0] = np.float32(t0 + slots + c)
        for s in range(wl.stream_steps):
            q = W.make(3, 60, (ft, h, d), "bf16", 1.0, c, s)
            k = W.make(3, 61, (ft, h, d), "bf16", 1.0, c, s)
            v = W.make(3, 62, (ft, h, d), "bf16", 1.0, c, s)
            st.attend(W.to_torch(q, dev), W.to_torch(k, dev), W.to_torch(v, dev), torch.from_numpy(cp).to(dev), O)
            torch.cuda.synchronize()
            rows = sorted(set(rng.choice(ft, min(16, ft), replace=False).tolist()) | {0, ft - 1})
            heads = sorted({0, h // 2, h - 1})
            want, kr = oc.attend(q.f32, k.f32, v.f32, cp, rows=rows, heads=heads)
            say("split stream chunk %d step %d" % (c, s))
            assert_parity(to_np(O)[rows][:, heads], want, "bf16", "split stream c%d s%d" % (c, s))
        st.append(c)
        oc.append(c, kr, v.f32)
