"""The oracle and the library stay apart (CPU only).

* Nothing in the library package (Python, HIP, C++) names the oracle, and
  the oracle imports nothing from the package, the header or the benchmark.
* The only shared module, ``workloads``, imports neither side.
* ``bench.py`` imports the oracle only inside ``cpu_baseline`` and
  ``__graft_entry__.py`` only inside ``smoke``.
* The binding has no fallback: without the built library it fails to import.
"""
import ast
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "multimodal_diffusion_transformer_amd")


def _files(top, exts):
    for d, dirs, files in os.walk(top):
        dirs[:] = [x for x in dirs if x not in ("__pycache__", "_build")]
        for f in files:
            if f.endswith(exts):
                yield os.path.join(d, f)


def _imported_modules(path, tree=None):
    if tree is None:
        tree = ast.parse(open(path, encoding="utf-8").read())
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name.split(".")[0], node
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            yield node.module.split(".")[0], node


def test_library_never_names_the_oracle():
    for path in _files(PKG, (".py", ".hip", ".cpp", ".hpp", ".h")):
        text = open(path, encoding="utf-8").read()
        assert "oracle" not in text, path
    assert "oracle" not in open(os.path.join(ROOT, "include", "motattn.h"), encoding="utf-8").read()


def test_oracle_imports_nothing_from_the_library():
    for path in _files(os.path.join(ROOT, "oracle"), (".py",)):
        mods = {m for m, _ in _imported_modules(path)}
        assert not mods & {"multimodal_diffusion_transformer_amd", "bench", "__graft_entry__",
                           "torch", "ctypes"}, path


def test_workloads_import_neither_side():
    for path in _files(os.path.join(ROOT, "workloads"), (".py",)):
        mods = {m for m, _ in _imported_modules(path)}
        assert not mods & {"oracle", "multimodal_diffusion_transformer_amd"}, path


@pytest.mark.parametrize("fname,allowed", [("bench.py", "cpu_baseline"),
                                           ("__graft_entry__.py", "smoke")])
def test_oracle_imported_only_where_allowed(fname, allowed):
    path = os.path.join(ROOT, fname)
    tree = ast.parse(open(path, encoding="utf-8").read())
    owners = {}
    for fn in ast.walk(tree):
        if isinstance(fn, (ast.FunctionDef, ast.AsyncFunctionDef)):
            for node in ast.walk(fn):
                owners.setdefault(id(node), fn.name)
    found = [(node, owners.get(id(node))) for m, node in _imported_modules(path, tree)
             if m == "oracle"]
    assert found, "expected the %s leg to use the oracle" % allowed
    for node, owner in found:
        assert owner == allowed, "%s imports the oracle at line %d, outside %s" % (fname, node.lineno,
                                                                                     allowed)


def test_binding_fails_without_the_library(tmp_path):
    pkg = tmp_path / "multimodal_diffusion_transformer_amd"
    pkg.mkdir()
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            shutil.copy(os.path.join(PKG, f), pkg / f)
    r = subprocess.run([sys.executable, "-c", "import multimodal_diffusion_transformer_amd"],
                       cwd=str(tmp_path), capture_output=True, text=True,
                       env=dict(os.environ, PYTHONPATH=str(tmp_path)))
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "not built" in r.stderr
