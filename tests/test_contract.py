"""Host-side checks of the product boundary: the package never reaches the
oracle, fails loudly without its HIP library, and the benchmark refuses a
multi-GPU run (one GPU only)."""
import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixed_precision_weight_page_amd")


def _imported_modules(path):
    tree = ast.parse(open(path).read(), filename=path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


def test_package_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            p = os.path.join(dirpath, f)
            if f.endswith(".py"):
                mods = list(_imported_modules(p))
                assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), (p, mods)
            elif f.endswith((".hip", ".cpp", ".h")):
                src = open(p).read()
                assert "oracle/" not in src and "oracle.py" not in src, p


def test_missing_library_fails_loudly(monkeypatch):
    from mixed_precision_weight_page_amd import pagedweight as pw
    monkeypatch.setattr(pw, "_LIB_PATH", os.path.join(ROOT, "no_such_dir", "libpagedweight.so"))
    monkeypatch.setattr(pw, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        pw.lib()


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpp_oracle_shares_nothing_with_the_library():
    """The plain C++ oracle includes only standard headers, and no library
    source or Python module of the package names it."""
    import re
    src = open(os.path.join(ROOT, "oracle", "cpu_oracle.cpp")).read()
    includes = re.findall(r'#include\s*[<"]([^>"]+)[>"]', src)
    assert includes and all(h in ("math.h", "stdint.h", "string.h", "vector") for h in includes), includes
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                assert "cpu_oracle" not in open(os.path.join(dirpath, f)).read(), f
