"""The oracle and the HIP path share nothing, and the product has no CPU
fallback (host only).

* no module of the package imports the oracle, and no oracle module imports
  the package;
* the HIP sources include no oracle file and the oracle's C source includes
  only standard headers;
* importing the package where its library is not built raises instead of
  falling back to anything.
"""
import ast
import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "deterministic_persistent_gemm_amd")
ORACLE = os.path.join(ROOT, "oracle")


def imported_modules(path):
    tree = ast.parse(open(path).read(), path)
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            names.add(node.module.split(".")[0])
    return names


def py_files(d):
    for dirpath, _, files in os.walk(d):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(dirpath, f)


def test_package_never_imports_the_oracle():
    for f in py_files(PKG):
        assert "oracle" not in imported_modules(f), f


def test_oracle_never_imports_the_package():
    for f in py_files(ORACLE):
        mods = imported_modules(f)
        assert "deterministic_persistent_gemm_amd" not in mods and "workloads" not in mods, f


def test_sources_share_no_headers():
    csrc = os.path.join(PKG, "csrc")
    for f in os.listdir(csrc):
        text = open(os.path.join(csrc, f), errors="replace").read()
        for inc in re.findall(r'#include\s+[<"]([^>"]+)[>"]', text):
            assert "oracle" not in inc, (f, inc)
    for f in os.listdir(ORACLE):
        if f.endswith((".c", ".h")):
            text = open(os.path.join(ORACLE, f)).read()
            for inc in re.findall(r'#include\s+[<"]([^>"]+)[>"]', text):
                assert inc in ("math.h", "stdint.h", "stdlib.h", "string.h", "omp.h", "stddef.h", "float.h"), (f, inc)


def test_import_without_the_library_raises(tmp_path):
    # a copy of the package's Python files without libbi.so
    dst = tmp_path / "deterministic_persistent_gemm_amd"
    dst.mkdir()
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            shutil.copy(os.path.join(PKG, f), dst / f)
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    r = subprocess.run([sys.executable, "-c", "import deterministic_persistent_gemm_amd"], cwd=str(tmp_path),
                       env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "not built" in r.stderr
