"""Builds the library's own kernel sources for the CPU SIMT emulator
(tests/native/emu) and calls them through the library's C ABI.

The sources are compiled unchanged except for the few inline-asm lines that
only a GPU assembler accepts, each replaced by the emulator call that does
what the instruction does (``SUBST``; every rule must match exactly the
number of times stated, so a change to the sources cannot slip past it).
"Device" buffers are host memory from ``emu_alloc``: each ends at a guard
page (or starts right after one), so a kernel read or write past either end
of a buffer ends the launch with a memory fault that the emulator reports.
"""
from __future__ import annotations

import concurrent.futures as cf
import ctypes
import os
import re
import subprocess

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "multimodal_diffusion_transformer_amd", "csrc")
EMU = os.path.join(ROOT, "tests", "native", "emu")
CXX = "/opt/rocm/llvm/bin/clang++"

# (pattern, replacement, {file: expected count})
SUBST = [
    (r'asm volatile\("s_nop \d\\n\\tglobal_load_lds_dwordx4 %0, %1" ::"v"\(voff\), "s"\(sb\), '
     r'"\{m0\}"\(lds\) : "memory"\);',
     "::emu::dma16(sb, voff, lds);", {"attention.hip": 1, "gemm.hip": 1}),
    (r'asm volatile\("s_waitcnt vmcnt\(0\)" ::: "memory"\);', "::emu::wait_vmem0();",
     {"attention.hip": 1, "gemm.hip": 1}),
    (r'asm volatile\("" ::"v"\(([^()]*(?:\([^()]*\))?[^()]*)\)\);', r"(void)(\1);", {"attention.hip": 1}),
    (r"\(uint32_t\)\(uintptr_t\)\(const __attribute__\(\(address_space\(3\)\)\) void\*\)p",
     "::emu::lds_offset(p)", {"attention.hip": 1, "gemm.hip": 1}),
    (r"__attribute__\(\(address_space\(3\)\)\) ", "", {"attention.hip": 1, "gemm.hip": 1}),
    (r"extern __shared__ __align__\(16\) unsigned char (\w+)\[\];",
     r"unsigned char* \1 = ::emu::lds_dynamic();", {"attention.hip": 1, "gemm.hip": 2}),
    (r"__attribute__\(\(amdgpu_waves_per_eu\(\d+, \d+\)\)\)", "", {"attention.hip": 1, "gemm.hip": 1}),
]


def transform(name: str, src: str) -> str:
    for pat, rep, counts in SUBST:
        src, n = re.subn(pat, rep, src)
        want = counts.get(name, 0)
        if n != want:
            raise RuntimeError("emulator rewrite %r matched %d times in %s, expected %d" % (pat, n, name, want))
    code = re.sub(r"//[^\n]*", "", src)
    if re.search(r"\basm\b|address_space", code):
        raise RuntimeError("%s still holds GPU-only code after the rewrite" % name)
    return src


UBSAN_LIB_DIR = "/opt/rocm/llvm/lib/clang/22/lib/linux"


def build(out_dir: str, dma_gemm: bool = False, jobs: int = 8, patches=(), ubsan=None) -> str:
    """Builds the emulated library in out_dir; `patches` are (file, old,
    new) text replacements applied first (to plant a mistake in a copy).
    With ubsan (default: the MOT_EMU_UBSAN environment variable) the kernel
    sources and the emulator are built with UndefinedBehaviorSanitizer,
    aborting at the first report."""
    if ubsan is None:
        ubsan = os.environ.get("MOT_EMU_UBSAN") == "1"
    os.makedirs(out_dir, exist_ok=True)
    # the sources include "../../include/motattn.h": keep that layout
    src_dir = os.path.join(out_dir, "pkg", "csrc")
    os.makedirs(src_dir, exist_ok=True)
    os.makedirs(os.path.join(out_dir, "include"), exist_ok=True)
    with open(os.path.join(ROOT, "include", "motattn.h")) as fh, \
            open(os.path.join(out_dir, "include", "motattn.h"), "w") as out:
        out.write(fh.read())
    for f in os.listdir(CSRC):
        text = open(os.path.join(CSRC, f)).read()
        for pf, old, rep in patches:
            if pf == f:
                if old not in text:
                    raise RuntimeError("patch text not found in %s: %r" % (f, old))
                text = text.replace(old, rep)
        if f.endswith(".hip"):
            text = transform(f, text)
        with open(os.path.join(src_dir, f), "w") as fh:
            fh.write(text)
    flags = ["-O2", "-fPIC", "-std=c++17", "-fno-strict-aliasing", "-w", "-I", EMU,
             "-I", os.path.join(ROOT, "include"), "-I", src_dir]
    if dma_gemm:
        flags.append("-DMOT_GEMM_DMA=1")
    link = []
    if ubsan:
        flags += ["-fsanitize=undefined", "-fno-sanitize-recover=all", "-g"]
        link = ["-fsanitize=undefined", "-shared-libsan", "-Wl,-rpath," + UBSAN_LIB_DIR]
    cmds, objs = [], []
    for f in sorted(os.listdir(src_dir)):
        if f.endswith((".hip", ".cpp")):
            o = os.path.join(out_dir, f + ".o")
            cmds.append([CXX, *flags, "-x", "c++", "-c", os.path.join(src_dir, f), "-o", o])
            objs.append(o)
    o = os.path.join(out_dir, "emu.o")
    cmds.append([CXX, *flags, "-c", os.path.join(EMU, "emu.cpp"), "-o", o])
    objs.append(o)

    def run(cmd):
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode:
            raise RuntimeError("emulator build failed: %s\n%s" % (" ".join(cmd), r.stderr[-4000:]))

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(run, cmds))
    lib = os.path.join(out_dir, "libmotattn_emu.so")
    run([CXX, "-shared", "-fPIC", "-o", lib, *objs, "-lpthread", *link])
    return lib


# emu_stat counters
ST_LAUNCH, ST_GROUPS, ST_DMA, ST_MFMA, ST_TR16, ST_BAR = range(6)


class Emu:
    """The emulated library: C ABI calls on guarded host buffers."""

    def __init__(self, path: str):
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.emu_alloc.restype = ctypes.c_void_p
        L.emu_alloc.argtypes = [ctypes.c_size_t, ctypes.c_int]
        L.emu_free.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
        L.emu_fault.restype = ctypes.c_char_p
        L.emu_config.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.emu_stat.restype = ctypes.c_uint64
        L.emu_stat.argtypes = [ctypes.c_int]
        L.emu_subset.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        # the C entry points take the argument types the product binding
        # declares for them
        from multimodal_diffusion_transformer_amd import _binding
        for name in _binding.EXPORTED:
            src, dst = getattr(_binding._lib, name), getattr(L, name)
            dst.restype = src.restype
            if src.argtypes is not None:
                dst.argtypes = src.argtypes
        self._bufs = []

    def config(self, dma_late=False, reverse_waves=False, threads=8):
        """reverse_waves: False / True, or 2 for a seeded random wave order in
        every phase between barriers."""
        self.lib.emu_config(int(dma_late), int(reverse_waves), int(threads))

    def subset(self, stride=0, offset=0, max_groups=0):
        """Run only workgroups offset, offset + stride, ... (at most
        max_groups) of the following launches; stride 0 runs all again."""
        self.lib.emu_subset(int(stride), int(offset), int(max_groups))

    def stat(self, i):
        return int(self.lib.emu_stat(i))

    def array(self, a, guard_front=False):
        """A guarded copy of numpy array `a` (C order)."""
        a = np.ascontiguousarray(a)
        n = max(a.nbytes, 1)
        p = self.lib.emu_alloc(n, int(guard_front))
        if not p:
            raise MemoryError("emu_alloc")
        self._bufs.append((p, n))
        buf = (ctypes.c_uint8 * n).from_address(p)
        out = np.frombuffer(buf, dtype=np.uint8, count=a.nbytes).view(a.dtype).reshape(a.shape)
        out[...] = a
        return out

    def empty(self, shape, dtype, guard_front=False):
        return self.array(np.zeros(shape, dtype), guard_front)

    def free_all(self):
        for p, n in self._bufs:
            self.lib.emu_free(ctypes.c_void_p(p), n)
        self._bufs = []

    def fault(self):
        return self.lib.emu_fault().decode()

    def call(self, fn, *args):
        """Calls C entry point `fn`; returns its status, raising on an
        emulator fault."""
        st = getattr(self.lib, fn)(*args)
        f = self.fault()
        if f:
            raise AssertionError("%s: %s" % (fn, f))
        return st


def ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)
