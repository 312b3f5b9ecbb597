"""Host-side checks of the attention kernels' gfx950 machine code in the
built library (our own build, read with the ROCm LLVM tools):

* the compiler's metadata: 64-lane waves, 256-lane workgroups, and at most
  256 VGPRs (arch + acc) per lane, so two waves fit on each SIMD;
* each step of the key loop is one branch-free run of NST x D/16 score and
  NST x 2 x ceil(D/32) PV MFMAs (NST = 2 tiles of 32 keys; D = 80: 10 and
  12) with no scratch access.  The
  D = 128 kernels spill a few registers; those accesses must stay in the
  cold paths (the overflow recompute).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "multimodal_diffusion_transformer_amd", "libmotattn.so")
LLVM = "/opt/rocm/llvm/bin"
KERNEL = "attn_fwd_mfma"

pytestmark = pytest.mark.skipif(
    not os.path.exists(LIB) or not os.path.exists(os.path.join(LLVM, "llvm-objdump")),
    reason="library not built or ROCm LLVM tools missing")


def _code_objects(tmp_path):
    fb = tmp_path / "fatbin"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", ".hip_fatbin=%s" % fb, LIB],
                   check=True)
    data = fb.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(b"__CLANG_OFFLOAD_BUNDLE__"), data)]
    out = []
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
        bundle = tmp_path / ("b%d" % n)
        bundle.write_bytes(data[a:b])
        co = tmp_path / ("b%d.co" % n)
        r = subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", "--input=%s" % bundle,
                            "--output=%s" % co], capture_output=True)
        if r.returncode == 0 and co.exists():
            out.append(co)
    return out


def _attention_code_object(tmp_path):
    for co in _code_objects(tmp_path):
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", str(co)],
                               capture_output=True, text=True, check=True).stdout
        if KERNEL in notes:
            return co, notes
    raise AssertionError("attention kernels not found in the build")


def _kernel_metadata(notes):
    """{kernel name: {key: value}} from the code object's AMDGPU metadata."""
    out = {}
    for block in re.split(r"\n\s*- \.", notes):
        m = re.search(r"\.name:\s+(\S+)", block)
        if not m or KERNEL not in m.group(1):
            continue
        kv = dict(re.findall(r"\.(\w+):\s+(\S+)", "." + block))
        out[m.group(1)] = kv
    return out


def test_attention_kernels_fit_two_waves_per_simd(tmp_path):
    _, notes = _attention_code_object(tmp_path)
    md = _kernel_metadata(notes)
    assert len(md) == 6, sorted(md)  # D = 64, 80, 128, each with and without Q rotation
    for name, kv in md.items():
        assert kv["wavefront_size"] == "64", name
        assert kv["max_flat_workgroup_size"] == "256", name
        assert int(kv["vgpr_count"]) + int(kv.get("agpr_count", "0")) <= 256, (name, kv["vgpr_count"])


def test_each_key_step_is_branch_free_and_spill_free(tmp_path):
    co, _ = _attention_code_object(tmp_path)
    dis = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", str(co)],
                         capture_output=True, text=True, check=True).stdout
    kernels, name = {}, None
    for line in dis.split("\n"):
        m = re.match(r"^[0-9a-f]+ <(.*)>:", line)
        if m:
            name = m.group(1)
            kernels[name] = [[]]
            continue
        m = re.match(r"^\s+(\S.*?)\s*// [0-9A-F]+:", line)
        if name is None or not m:
            continue
        text = m.group(1)
        if re.match(r"s_(c)?branch|s_setpc|s_endpgm", text):
            kernels[name].append([])  # a new branch-free run
        else:
            kernels[name][-1].append(text)
    checked = 0
    for name, runs in kernels.items():
        if KERNEL not in name:
            continue
        d = int(re.search(r"ILi(\d+)E", name).group(1))
        per_step = 2 * (d // 16) + 2 * 2 * ((d + 31) // 32)  # NST = 2: score and PV MFMAs
        steps = [r for r in runs if sum(t.startswith("v_mfma") for t in r) == per_step]
        # the two steps of the unrolled key loop, each one branch-free run
        assert len(steps) >= 2, (name, [sum(t.startswith("v_mfma") for t in r) for r in runs if r])
        for r in steps:
            spill = [t for t in r if t.startswith("scratch_") or t.startswith("buffer_")]
            assert not spill, (name, spill[:5])
        checked += 1
    assert checked == 6


def _all_kernel_metadata(tmp_path):
    out = {}
    for co in _code_objects(tmp_path):
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", str(co)],
                               capture_output=True, text=True, check=True).stdout
        for block in re.split(r"\n\s*- \.", notes):
            m = re.search(r"\.name:\s+(\S+)", block)
            if m:
                out[m.group(1)] = dict(re.findall(r"\.(\w+):\s+(\S+)", "." + block))
    return out


# the bandwidth-bound kernels and the region GEMM: no scratch spills; the
# HBM-bound kernels keep at least 4 waves per SIMD (<= 128 VGPRs), except the
# LayerNorm instance for rows past 4,096 columns, which holds 16 chunks of
# 16 bytes per lane in registers (2 waves per SIMD, 16 loads in flight each)
NO_SPILL = ("layernorm_kernel", "attn_merge_kernel", "euler_kernel", "mrope_kernel", "gemm_region_bf16")
HBM_BOUND = ("layernorm_kernel", "attn_merge_kernel", "euler_kernel", "mrope_kernel")


def test_other_kernels_spill_free(tmp_path):
    md = _all_kernel_metadata(tmp_path)
    seen = set()
    for name, kv in md.items():
        hit = [k for k in NO_SPILL if k in name]
        if not hit:
            continue
        seen |= set(hit)
        assert int(kv.get("private_segment_fixed_size", "0")) == 0, (name, kv.get("private_segment_fixed_size"))
        if any(k in name for k in HBM_BOUND):
            limit = 256 if "layernorm_kernelILi16E" in name else 128
            assert int(kv["vgpr_count"]) <= limit, (name, kv["vgpr_count"])
    assert seen == set(NO_SPILL), sorted(seen)
