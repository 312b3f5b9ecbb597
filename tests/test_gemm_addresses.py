"""Every LDS-DMA copy and operand read of the direct-to-LDS region GEMM,
checked on the CPU (no GPU).  That kernel is built only on request
(-DMOT_GEMM_DMA=1) until it has run on a GPU; these checks come first.

tests/native/gemm_addr_check.hip includes the header the kernel uses
(csrc/gemm_tiles.hpp) and walks, for a problem (rows [r0, r0 + rows) of
X [M, K], weights W [K, N]), the copies of the first two and last two tiles
in each direction and stage (all of them for small problems; the addresses
are affine in the tile and stage indices): no lane offset wraps, every copy
reads exactly the 8-element run of X or W its slot needs inside the matrix,
each LDS slot is written once at its swizzled chunk, and the MFMA operand
reads give the rows, columns and k the output they feed needs.

Problems: both rooms of every workload's QKV and output projections, the
guided step's two-prediction output projection, the whole layer's MLP
matrices, and ragged rows and columns.  Planted mistakes in a copy of the
header must make the walk fail.
"""
import os
import subprocess

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "multimodal_diffusion_transformer_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "gemm_addr_check.hip")
HIPCC = "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="ROCm compiler missing")


def _build(out, inc=CSRC):
    subprocess.run([HIPCC, "-x", "hip", "--cuda-host-only", "-O2", "-std=c++17", "-I", inc,
                    "-I", os.path.join(ROOT, "include"), SRC, "-o", str(out)],
                   check=True, capture_output=True)


def _run(exe, problems):
    args = [str(a) for p in problems for a in p]
    r = subprocess.run([str(exe), *args], capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout


def _rooms(M, K, N, n_ar):
    """The two problems of one region-split launch: (M, K, N, r0, rows)."""
    out = []
    if n_ar > 0:
        out.append((M, K, N, 0, n_ar))
    if n_ar < M:
        out.append((M, K, N, n_ar, M - n_ar))
    return out


def _workload_problems():
    probs = []
    for wl in W.WORKLOADS:
        if wl.dtype != "bf16" or wl.mask != W.AR_CAUSAL_DM_FULL:
            continue
        n, hid, h, d, hk = wl.n_tokens, wl.hidden, wl.n_heads, wl.head_dim, wl.kv_heads
        n_ar = W.region_counts(wl.segments)[0]
        probs += _rooms(n, hid, (h + 2 * hk) * d, n_ar)   # QKV
        probs += _rooms(n, h * d, hid, n_ar)              # output projection
        if wl.ffn:
            probs += _rooms(n, hid, wl.ffn, n_ar)         # MLP up
            probs += _rooms(n, wl.ffn, hid, n_ar)         # MLP down
        n_dm = n - n_ar
        probs.append((2 * n_dm, h * d, hid, 0, 2 * n_dm))  # the guided step's O projection
    return probs


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = tmp_path_factory.mktemp("gac") / "gemm_addr_check"
    _build(out)
    return out


@pytest.mark.parametrize("prob", _workload_problems(), ids=lambda p: "M%d_K%d_N%d_r%d_%d" % p)
def test_workload_problems(exe, prob):
    rc, out = _run(exe, [prob])
    assert rc == 0 and out.startswith("ok"), out


def test_ragged_problems(exe):
    probs = []
    for rows, n_ar, K, N in [(300, 130, 256, 384), (260, 70, 64, 192), (1, 1, 32, 64), (257, 0, 96, 64),
                             (511, 255, 64, 320), (700, 0, 32, 1152)]:
        probs += _rooms(rows, K, N, n_ar)
    rc, out = _run(exe, probs)
    assert rc == 0 and out.startswith("ok"), out


PLANTED = [
    ("ragged X rows not clamped", "if (row > rows - 1) row = rows - 1;", ""),
    ("ragged W chunks not clamped", "if (c > last_c) c = last_c;", ""),
    ("W copy without the swizzle its reads apply",
     "static int w_chunk(int row, int lane) { return (lane % 16) ^ (4 * (row & 3)); }",
     "static int w_chunk(int row, int lane) { return (lane % 16); }"),
    ("X read without the swizzle", "((g ^ ((l32 >> 2) & 1)) * 16)", "((g) * 16)"),
    ("W load rows off by one load", "return (int64_t)4 * i * N * 2;", "return (int64_t)4 * (i + 1) * N * 2;"),
    ("A operand columns of the other block", "const int c = 8 * wn + 4 * nb + 2 * q16 + (j & 3) / 2;",
     "const int c = 8 * wn + 4 * (1 - nb) + 2 * q16 + (j & 3) / 2;"),
]


@pytest.mark.parametrize("what,pat,rep", PLANTED, ids=[p[0] for p in PLANTED])
def test_planted_mistake_is_caught(tmp_path, what, pat, rep):
    src = open(os.path.join(CSRC, "gemm_tiles.hpp")).read()
    assert pat in src, what
    inc = tmp_path / "inc"
    inc.mkdir()
    (inc / "gemm_tiles.hpp").write_text(src.replace(pat, rep))
    out = tmp_path / "gac"
    _build(out, str(inc))
    rc, text = _run(out, _rooms(300, 256, 384, 130) + _rooms(260, 64, 192, 70))
    assert rc != 0 and "FAIL" in text, what
