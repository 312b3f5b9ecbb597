"""The kernel sources on the CPU emulator built with UndefinedBehaviorSanitizer
(signed overflow, invalid shifts, misaligned or null accesses, out-of-range
conversions in the kernels' index and arithmetic code abort with a report).
The emulator parity tests run in a child process on that build; a planted
overflow in a copy of a kernel must be reported.
"""
import ctypes
import os
import subprocess
import sys

import pytest

from tests import emu_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not (os.path.exists(emu_lib.CXX) and os.path.isdir(emu_lib.UBSAN_LIB_DIR)),
                                reason="host clang++ or its sanitizer runtime missing")


def test_kernel_parity_tests_under_ubsan():
    pytest.importorskip("multimodal_diffusion_transformer_amd._binding")
    env = dict(os.environ, MOT_EMU_UBSAN="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_emu_kernels.py", "-q", "-p", "no:cacheprovider",
                        "-k", "not planted and not dma_late_rev"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out, out[-4000:]


PLANT = ("euler.hip", "const int64_t stride = (int64_t)gridDim.x * blockDim.x;",
         "const int64_t stride = (int64_t)gridDim.x * blockDim.x;"
         " { volatile int big = 2147483647; volatile int o = big + (int)threadIdx.x; (void)o; }")

CHILD = r"""
import ctypes, sys
import numpy as np
sys.path.insert(0, %r)
from tests import emu_lib
E = emu_lib.Emu(%r)
X = E.array(np.zeros(64, np.float32)); V = E.array(np.zeros(64, np.float32))
E.call("flow_euler_step", emu_lib.ptr(X), emu_lib.ptr(V), 1, 64, ctypes.c_float(1), ctypes.c_float(0.5), None, None)
"""


def test_planted_overflow_is_reported(tmp_path):
    pytest.importorskip("multimodal_diffusion_transformer_amd._binding")
    lib = emu_lib.build(str(tmp_path / "b"), ubsan=True, patches=[PLANT])
    r = subprocess.run([sys.executable, "-c", CHILD % (ROOT, lib)], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0 and "signed integer overflow" in r.stderr, r.stderr[-2000:]
