"""Host-side rules of the product path (CPU only, no kernel launched).

* The binding fails loudly when libbsa.so is missing: there is no CPU fallback.
* The oracle and the HIP path share no code: no product module imports or includes the oracle,
  and the oracle imports only numpy and the standard library.
* bench.py measures one GPU and refuses a larger --gpus with a message.
"""
import ast
import os
import subprocess
import sys

import pytest

from video_dit_block_cube_amd import bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "video_dit_block_cube_amd")


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(bsa, "LIB_PATH", str(tmp_path / "libbsa.so"))
    monkeypatch.setattr(bsa, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        bsa.lib()
    p = bsa.Problem(1, 1, 64, 4, 8, 8, 2, 4, 4)
    with pytest.raises(RuntimeError, match="not built"):
        bsa.bsa_num_selected(p, 2)


def _imports(path):
    tree = ast.parse(open(path, encoding="utf-8").read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            if node.level:
                names.add("." + (node.module or ""))
            elif node.module:
                names.add(node.module.split(".")[0])
    return names


def test_product_never_imports_the_oracle():
    for name in os.listdir(PKG):
        full = os.path.join(PKG, name)
        if name.endswith(".py"):
            assert "oracle" not in _imports(full), name
    csrc = os.path.join(PKG, "csrc")
    for name in os.listdir(csrc):
        text = open(os.path.join(csrc, name), encoding="utf-8").read()
        assert "oracle" not in text.lower(), name


def test_oracle_imports_only_numpy_and_the_standard_library():
    allowed = {"__future__", "math", "dataclasses", "functools", "numpy", "itertools", "typing",
               ".bsa_oracle", ".prologue", "."}
    odir = os.path.join(ROOT, "oracle")
    for name in os.listdir(odir):
        if name.endswith(".py"):
            extra = _imports(os.path.join(odir, name)) - allowed
            assert not extra, (name, extra)


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stdout + res.stderr
