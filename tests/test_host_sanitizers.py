"""The library's host-side code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU).

The library's sources are rebuilt with the sanitizers on their host side
only (the device code is built as usual, and no kernel is launched) and
linked with
tests/native/host_sanitize.cpp, which drives the packed-sequence layout
(the five workloads, rejected orders, counts and frame / step indices at and
past the int64 limit), the noise schedule over a sweep of step counts and
shifts, the host tile classifier, and the argument checks of every device
entry point with arguments each check must reject before any launch.  Any
sanitizer report aborts the program.
"""
import concurrent.futures as cf
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "multimodal_diffusion_transformer_amd", "csrc")
INC = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="ROCm compilers missing")

COMMON = ["-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-std=c++17", "-I", INC]
# the HIP sources: host side only, sanitizers on the host side
HIP_HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
# plain C++ sources and the link
CXX_SAN = ["-fsanitize=address,undefined"]


def _sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    hip, cpp = _sources()
    objs = []
    cmds = []
    for f in hip:
        o = d / (f + ".o")
        cmds.append([HIPCC, "--offload-arch=gfx950", *COMMON, *HIP_HOST_SAN, "-Xclang", "-target-feature",
                     "-Xclang", "-packed-fp32-ops", "-c", os.path.join(CSRC, f), "-o", str(o)])
        objs.append(str(o))
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        for r in ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds):
            assert r.returncode == 0, r.stdout + r.stderr
    for f in cpp:
        o = d / (f + ".o")
        subprocess.run([CLANG, *COMMON, "-ffp-contract=off", *CXX_SAN, "-c", os.path.join(CSRC, f),
                        "-o", str(o)], check=True, capture_output=True)
        objs.append(str(o))
    main = d / "main.o"
    subprocess.run([CLANG, *COMMON, *CXX_SAN, "-c", os.path.join(ROOT, "tests", "native", "host_sanitize.cpp"),
                    "-o", str(main)], check=True, capture_output=True)
    exe = d / "host_sanitize"
    subprocess.run([CLANG, *CXX_SAN, str(main), *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)], check=True, capture_output=True)
    return exe


def test_host_code_is_clean_under_asan_and_ubsan(program):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")
    r = subprocess.run([str(program)], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.stdout.startswith("ok"), out[-4000:]
