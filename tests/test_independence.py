"""The product path and the oracle are independent, and the product never falls back to the CPU.

* the package (Python binding and HIP / C++ sources) neither imports nor includes anything of
  the oracle, and names no oracle module;
* the oracle imports neither the package nor the library;
* the shared input generators import neither side;
* with the library missing, the binding raises instead of computing anything on the host.
"""
import ast
import importlib
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "optimizer_step_weight_amd")


def _files(top, exts):
    for d, _, names in os.walk(top):
        if "__pycache__" in d:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(d, n)


def _imported_modules(path):
    tree = ast.parse(open(path).read(), path)
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.level == 0 and node.module:
            mods.add(node.module.split(".")[0])
    return mods


def test_package_does_not_use_the_oracle():
    for f in _files(PKG, (".py",)):
        assert "oracle" not in _imported_modules(f), f"{f} imports the oracle"
        assert "oracle" not in open(f).read(), f"{f} names the oracle"
    for f in _files(os.path.join(PKG, "csrc"), (".hip", ".h", ".cpp")):
        src = open(f).read()
        for inc in re.findall(r'#include\s+[<"]([^>"]+)[>"]', src):
            assert "oracle" not in inc, f"{f} includes {inc}"


def test_oracle_does_not_use_the_package():
    for f in _files(os.path.join(ROOT, "oracle"), (".py",)):
        mods = _imported_modules(f)
        assert "optimizer_step_weight_amd" not in mods and "ctypes" not in mods, f
        assert "libforge" not in open(f).read(), f


def test_input_generators_import_neither_side():
    for f in _files(os.path.join(ROOT, "synth"), (".py",)):
        mods = _imported_modules(f)
        assert not mods & {"oracle", "optimizer_step_weight_amd"}, f"{f} imports {mods}"


def test_missing_library_raises(monkeypatch):
    forge = importlib.import_module("optimizer_step_weight_amd")
    monkeypatch.setattr(forge, "LIB_PATH", os.path.join(ROOT, "_no_such_dir", "libforge.so"))
    monkeypatch.setattr(forge, "_lib_handle", None)
    with pytest.raises(ImportError):
        forge._lib()
    X = torch.zeros((32, 128), dtype=torch.bfloat16)
    dY = torch.zeros((32, 128), dtype=torch.bfloat16)
    W = torch.zeros((128, 128), dtype=torch.bfloat16)
    with pytest.raises(ImportError):  # no host fallback computes the step
        forge.wgrad_step(X, dY, W, opt="sgd", hyper={"lr": 1.0}, step=1, seed=0)
    assert not W.any()
