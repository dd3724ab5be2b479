"""CPU checks that the oracle and the HIP path stay apart.

* No module of the package (the binding, the build script, the seeded input generators) imports the oracle,
  and no HIP source or public header refers to it.
* The oracle imports nothing but numpy, the standard library and its own modules.
* bench.py imports the oracle only in its CPU-baseline leg: inside the oracle step functions, the
  cpu_baseline function, or a block guarded by the cpu_needed flag that --no-cpu-baseline clears.
* Without the built library the binding raises instead of computing anything.
"""

import ast
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_fp4_kv_amd")


def _imports(tree):
    """(module name, node) for every import statement in the tree."""
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name, node
        elif isinstance(node, ast.ImportFrom):
            yield ("." * node.level) + (node.module or ""), node


def _parse(path):
    with open(path) as f:
        return ast.parse(f.read(), path)


def test_package_never_imports_the_oracle():
    files = glob.glob(os.path.join(PKG, "**", "*.py"), recursive=True)
    assert files
    for path in files:
        tree = _parse(path)
        for name, _ in _imports(tree):
            assert name.split(".")[0] != "oracle", f"{path} imports {name}"
        for node in ast.walk(tree):  # importlib / __import__ by name
            if isinstance(node, ast.Constant) and isinstance(node.value, str):
                assert not node.value.startswith("oracle"), f"{path} names {node.value!r}"


def test_hip_sources_and_headers_do_not_refer_to_the_oracle():
    files = (glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*.h")))
    assert files
    for path in files:
        with open(path, errors="replace") as f:
            text = f.read()
        assert "oracle/" not in text and '#include "oracle' not in text, path


def test_oracle_imports_only_numpy_and_itself():
    allowed = {"numpy", "math", "fractions", "functools", "itertools"}
    for path in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        for name, _ in _imports(_parse(path)):
            if name.startswith("."):
                continue
            assert name.split(".")[0] in allowed, f"{path} imports {name}"


def _guarded(node, parents):
    """True when an import node sits in the bench's CPU-baseline leg."""
    p = parents.get(node)
    while p is not None:
        if isinstance(p, ast.FunctionDef) and (p.name.startswith("oracle_") or p.name.startswith("_oracle")
                                               or p.name == "cpu_baseline"):
            return True
        if isinstance(p, ast.If) and "cpu_needed" in ast.unparse(p.test):
            return True
        p = parents.get(p)
    return False


def test_bench_imports_the_oracle_only_in_its_cpu_baseline_leg():
    tree = _parse(os.path.join(ROOT, "bench.py"))
    parents = {}
    for node in ast.walk(tree):
        for child in ast.iter_child_nodes(node):
            parents[child] = node
    found = 0
    for name, node in _imports(tree):
        if name.split(".")[0] == "oracle":
            found += 1
            assert _guarded(node, parents), f"bench.py line {node.lineno}: oracle import outside the CPU leg"
    assert found > 0  # the CPU baseline leg exists


def test_binding_raises_without_the_library():
    code = ("from sparse_attention_fp4_kv_amd import csa2\n"
            "csa2.LIB_PATH = '/nonexistent/libcsa2.so'\n"
            "csa2._LIB = None\n"
            "try:\n"
            "    csa2.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised:") and "not built" in r.stdout
