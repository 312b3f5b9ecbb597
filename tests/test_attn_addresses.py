"""Every LDS-DMA copy and LDS operand read of the bf16 attention kernel,
checked on the CPU (no GPU).

tests/native/attn_addr_check.hip includes the header the kernel's loader
uses (csrc/attn_tiles.hpp) and walks every copy of every K and V tile of
every head of a K/V view: each lane's unsigned 32-bit offset must not wrap,
scalar base + offset must be exactly the run of 8 dims of the key, head and
chunk that tile row needs (rows past the last key re-read the last key), each
LDS slot is written once at the swizzled chunk, and the K and transposed V
operand reads must give the keys and dims the MFMA layouts expect.  The walk
covers every tile index up to ceil(nk / 64), so it covers every launch of
that view in both mask modes and at any q0 and nq.

Views: the workloads (K and V as strided views of the packed
[N, 3, H, D] projection output; the streaming cache contiguous), ragged key
counts around the tile size, head-major layouts, and the largest token
stride the API accepts (64-row tiles below 4 GiB).  Planted mistakes in a
copy of the header must make the walk fail.
"""
import os
import re
import shutil
import subprocess

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "multimodal_diffusion_transformer_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "attn_addr_check.hip")
HIPCC = "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="ROCm compiler missing")

# the API's limit: a 64-row tile of K or V spans less than 4 GiB
MAX_TS = ((1 << 32) // 128 - 1) // 8 * 8


def _build(out, inc=CSRC):
    subprocess.run([HIPCC, "-x", "hip", "--cuda-host-only", "-O2", "-std=c++17", "-I", inc,
                    "-I", os.path.join(ROOT, "include"), SRC, "-o", str(out)],
                   check=True, capture_output=True)


def _full(v):
    """(D, nk, ts, hs, H) -> one batch item in a buffer that ends at the view."""
    d, nk, ts, hs, h = v
    return (d, nk, ts, hs, h, 1, 0, (nk - 1) * ts + (h - 1) * hs + d)


def _run(exe, views, maps=()):
    args = [str(a) for m in maps for a in ("map", *m)]
    args += [str(a) for v in views for a in (v if len(v) == 8 else _full(v))]
    r = subprocess.run([str(exe), *args], capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout


def _workload_views():
    views = []
    for wl in W.WORKLOADS:
        if wl.dtype != "bf16":
            continue
        h, d = wl.n_heads, wl.head_dim
        if wl.mask == W.CHUNK_CAUSAL_KV:
            ft = wl.stream_views * wl.stream_gh * wl.stream_gw
            nk = wl.stream_text + 2 + (wl.stream_history_frames + 1) * ft
            views.append((d, nk, h * d, d, h))          # the rolling cache [nk, H, D]
        else:
            hk = wl.kv_heads  # K or V of the fused [N, (H + 2 H_kv) D] projection output
            views.append((d, wl.n_tokens, (h + 2 * hk) * d, d, hk))
    return views


EDGE_NK = [1, 2, 63, 64, 65, 127, 128, 129, 300, 1030]


def _edge_views():
    v = []
    for d in (64, 80, 128):
        for nk in EDGE_NK:
            v.append((d, nk, 3 * 2 * d, d, 2))      # packed, 2 heads
            v.append((d, nk, 3 * d, d, 1))          # packed, 1 head
            v.append((d, nk, d, nk * d, 2))         # head-major [H][nk][D]
        v.append((d, 70, MAX_TS, d, 1))             # largest token stride accepted
        v.append((d, 129, MAX_TS, 8, 2))
    return v


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = tmp_path_factory.mktemp("aac") / "attn_addr_check"
    _build(out)
    return out


def test_max_stride_is_the_apis_limit():
    # the API rejects 64 * max(k_ts, v_ts) * 2 >= 2^32 (bf16); MAX_TS is the
    # largest stride that passes, rounded to the 8-element alignment
    assert 64 * MAX_TS * 2 < (1 << 32) <= 64 * (MAX_TS + 8) * 2


@pytest.mark.parametrize("view", _workload_views(), ids=lambda v: "d%d_nk%d_ts%d" % v[:3])
def test_workload_views(exe, view):
    rc, out = _run(exe, [view])
    assert rc == 0 and out.startswith("ok"), out


def _cfg_view(wl):
    """The guided step's K (or V) view: one packed [n_ar + n_dm + n_ar, 3, H, D]
    buffer holding [AR cond | DM | AR base]; item 0 reads rows [0, N), item 1
    rows [n_ar, n_ar + N)."""
    n_ar = W.region_counts(wl.segments)[0]
    n = wl.n_tokens
    h, d = wl.n_heads, wl.head_dim
    ts = 3 * h * d
    rows = n + n_ar
    # K starts at element h*d of the buffer; the extent is counted from there
    return (d, n, ts, d, h, 2, n_ar * ts, rows * ts - h * d)


@pytest.mark.parametrize("name", ["policy_bf16", "t2v480p_bf16"])
def test_guided_pair_views(exe, name):
    rc, out = _run(exe, [_cfg_view(W.BY_NAME[name])])
    assert rc == 0 and out.startswith("ok"), out


def test_grouped_heads_and_batches(exe):
    d = 128
    views = [
        (d, 300, (32 + 16) * d, d, 8, 1, 0, 299 * 48 * d + 8 * d),  # 32/8-head K of a fused QKV row
        (d, 129, 8 * d, d, 8, 3, 129 * 8 * d, 3 * 129 * 8 * d),                # 3 items, contiguous
        (d, 70, d, 70 * d, 2, 2, 2 * 70 * d, 4 * 70 * d),                       # head-major, 2 items
        (64, 65, 2 * 64, 64, 2, 2, 0, 64 * 64 * 2 + 64 * 2),                    # one K shared by 2 items
    ]
    rc, out = _run(exe, views, maps=[(24, 1), (32, 4), (16, 2), (64, 8), (8, 8), (6, 3), (40, 5)])
    assert rc == 0 and out.startswith("ok"), out


def test_edge_views(exe):
    rc, out = _run(exe, _edge_views())
    assert rc == 0 and out.startswith("ok"), out


PLANTED = [
    # (what, pattern, replacement) applied to a copy of attn_tiles.hpp
    ("ragged rows not clamped", "const int64_t rr = r > last ? last : r;", "const int64_t rr = r;"),
    ("K copy without the swizzle the reads apply",
     "return (lane % L::CH) ^ (IS_K ? swz_k<DS>(r) : swz_v<DS>(r));",
     "return (lane % L::CH) ^ (IS_K ? 0 : swz_v<DS>(r));"),
    ("V swizzle ignored by the reads", "const int f = swz_v<D>(rowl);", "const int f = 0;"),
    ("row within a load off by one chunk", "return (wave * PER_WAVE + i) * L::RPI + lane / L::CH;",
     "return (wave * PER_WAVE + i) * L::RPI + lane / L::CH + (lane == 63);"),
    ("key_perm halves swapped", "16 * ((rho >> 2) & 1)", "16 * (1 - ((rho >> 2) & 1))"),
    ("row bytes in 16-bit arithmetic", "return (uint32_t)(L::RPI * ts * 2);",
     "return (uint32_t)(uint16_t)(L::RPI * ts * 2);"),
    ("D = 80 padding chunks copied from past the row", "else return c < D / 8 ? c : c - D / 8;",
     "else return c;"),
    ("head slots not spread by XCD", "return xcd_heads ? (hs & 7) * xcd_heads + (hs >> 3) : hs;",
     "return xcd_heads ? (hs % xcd_heads) * 8 + hs / xcd_heads : hs;"),
]


@pytest.mark.parametrize("what,pat,rep", PLANTED, ids=[p[0] for p in PLANTED])
def test_planted_mistake_is_caught(tmp_path, what, pat, rep):
    src = open(os.path.join(CSRC, "attn_tiles.hpp")).read()
    assert pat in src, what
    inc = tmp_path / "inc"
    inc.mkdir()
    (inc / "attn_tiles.hpp").write_text(src.replace(pat, rep))
    out = tmp_path / "aac"
    _build(out, str(inc))
    views = [(128, 300, 9216, 128, 2), (64, 129, 768, 64, 2), (128, 70, MAX_TS, 128, 1), (80, 300, 6400, 80, 2)]
    rc, text = _run(out, views, maps=[(32, 4)])
    assert rc != 0 and "FAIL" in text, what
