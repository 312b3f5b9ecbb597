"""The GPU test files themselves, run on the CPU through the emulated library
(tests/emu_plugin.py): the tests' own inputs, layouts, oracle calls and
tolerances, the binding's marshalling and pipeline.py, against the product
kernel sources, with no GPU.  Cases too large for the emulator (the policy,
480p and full streaming shapes) are left out here; they run on a GPU, and
were run on the emulator by hand with the same plugin.  The streaming
rollouts run here at their reduced size, through the ring wrap.
"""
import os
import subprocess
import sys

import pytest

from tests import emu_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SLOW = ["long", "480p", "full", "bench", "sizes", "policy_bf16", "policy_shape", "stream_chunk_bf16", "4423681",
        "policy_layout"]


@pytest.mark.skipif(not os.path.exists(emu_lib.CXX), reason="host clang++ missing")
def test_gpu_suite_on_the_emulator(tmp_path):
    pytest.importorskip("torch")
    pytest.importorskip("multimodal_diffusion_transformer_amd._binding")
    env = dict(os.environ, MOT_EMU_LIB=emu_lib.build(str(tmp_path / "emu")))
    sel = " and ".join("not " + s for s in SLOW)
    r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-m", "gpu", "-p", "tests.emu_plugin", "-q",
                        "-k", sel, "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    tail = "\n".join(r.stdout.splitlines()[-30:])
    assert r.returncode == 0, tail
    assert " passed" in tail and "failed" not in tail, tail
