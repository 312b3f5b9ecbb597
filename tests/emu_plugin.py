"""pytest plugin: run the GPU tests on the CPU, through the library's kernel
sources built for the SIMT emulator (tests/emu_lib.py).

    python -m pytest tests -m gpu -p tests.emu_plugin -k "<cases>"

The product binding's C library handle is pointed at the emulated build,
its device checks accept CPU tensors and its stream is 0; the tests'
device() is the CPU and torch.cuda.synchronize() does nothing (every
emulated launch is synchronous).  Everything else (the binding's
marshalling, pipeline.py, the tests' own code and tolerances) runs as on a
GPU.  On the CPU, .to("cpu") and torch.from_numpy() alias instead of
copying, so the tests' conversions are made to copy.  The emulator is slow
(minutes per billion MACs), so select the small cases with -k.
"""
import ctypes
import os
import tempfile

import numpy as np


def pytest_configure(config):
    import torch

    from tests import emu_lib
    import tests.gpu_util as gu
    import workloads as W
    from multimodal_diffusion_transformer_amd import _binding as B

    path = os.environ.get("MOT_EMU_LIB") or emu_lib.build(tempfile.mkdtemp(prefix="mot_emu_"))
    emu = emu_lib.Emu(path)
    emu.config(dma_late=os.environ.get("MOT_EMU_DMA_LATE", "1") == "1",
               reverse_waves=os.environ.get("MOT_EMU_REVERSE", "1") == "1",
               threads=int(os.environ.get("MOT_EMU_THREADS", "8")))
    real_lib = B._lib

    class _Checked:
        """The emulated library; a call that ends in an emulator fault
        raises with the emulator's report."""

        def __getattr__(self, name):
            fn = getattr(emu.lib, name)

            def call(*a):
                st = fn(*a)
                f = emu.fault()
                if f:
                    raise AssertionError("%s: %s" % (name, f))
                return st
            return call

    assert real_lib is not None
    B._lib = _Checked()
    B._need_cuda = lambda *ts: None
    B._stream = lambda s: ctypes.c_void_p(0)
    gu.device = lambda: torch.device("cpu")
    torch.cuda.synchronize = lambda *a, **k: None
    orig_np = W.to_numpy_f32
    W.to_numpy_f32 = lambda t: np.array(orig_np(t), copy=True)
    gu.to_np = lambda t: W.to_numpy_f32(t)
    orig_tt = W.to_torch
    W.to_torch = lambda t, device=None: orig_tt(t, device).clone()
    config._mot_emu = emu
