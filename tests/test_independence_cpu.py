"""The HIP path and the oracle share no code (CPU, static checks of the sources).

- the library's sources include only their own headers (csrc/, include/) and
  system headers;
- the Python package (binding, build script, input generator) never imports
  the oracle, and the oracle imports nothing of the package or the library:
  only the standard library, numpy and its own modules;
- the C oracle includes only C library headers and is compiled from its own
  file alone;
- bench.py imports the oracle only inside its CPU-baseline functions, and
  __graft_entry__.py only inside build() (which compiles the C oracle, the
  checker, without running it) and smoke().
Only the seeded input generator (gr_kan_rational_amd/synth.py) serves both
sides; it is imported by the tests and bench.py, never by the oracle.
"""
from __future__ import annotations

import ast
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gr_kan_rational_amd")
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
ORACLE = os.path.join(ROOT, "oracle")

SYSTEM_HEADERS = {"hip/hip_runtime.h", "hip/hip_runtime_api.h", "stdint.h", "stddef.h", "limits.h",
                  "cstdlib", "mutex", "type_traits"}
C_LIBRARY_HEADERS = {"math.h", "float.h", "stddef.h", "stdio.h", "stdlib.h"}
ORACLE_PY_IMPORTS = {"__future__", "ctypes", "math", "os", "subprocess", "threading", "concurrent",
                     "numpy"}


def _py_files(d):
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".py"))


def _imports(path):
    """(module, level, enclosing function or None) for each import in the file."""
    tree = ast.parse(open(path).read(), path)
    out = []

    def visit(node, func):
        for child in ast.iter_child_nodes(node):
            if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)):
                visit(child, child.name if func is None else func)
                continue
            if isinstance(child, ast.Import):
                out.extend((a.name, 0, func) for a in child.names)
            elif isinstance(child, ast.ImportFrom):
                out.append((child.module or "", child.level, func))
            visit(child, func)

    visit(tree, None)
    return out


def _includes(path):
    return re.findall(r'^\s*#\s*include\s*([<"])([^>"]+)[>"]', open(path).read(), re.M)


def test_library_sources_include_only_their_own_and_system_headers():
    own = set(os.listdir(CSRC)) | set(os.listdir(INCLUDE))
    sources = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".h"))]
    sources += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    assert len(sources) >= 10
    for path in sources:
        for kind, name in _includes(path):
            if kind == '"':
                assert name in own, (path, name)
            else:
                assert name in SYSTEM_HEADERS, (path, name)
            assert "oracle" not in name, (path, name)


def test_package_never_imports_the_oracle():
    files = _py_files(PKG)
    assert any(f.endswith("binding.py") for f in files)
    for path in files:
        for mod, level, _ in _imports(path):
            assert level > 0 or mod.split(".")[0] != "oracle", (path, mod)
            assert "oracle" not in mod.split("."), (path, mod)


def test_oracle_imports_nothing_of_the_package_or_the_library():
    for path in _py_files(ORACLE):
        for mod, level, _ in _imports(path):
            if level > 0:
                continue  # the oracle's own modules
            assert mod.split(".")[0] in ORACLE_PY_IMPORTS, (path, mod)
        text = open(path).read()
        assert "libgrkan.so" not in text and "gr_kan_rational_amd" not in text, path


def test_c_oracle_is_built_from_its_own_file_alone():
    c_files = [f for f in os.listdir(ORACLE) if f.endswith((".c", ".h"))]
    assert c_files == ["grkan_oracle.c"]
    for kind, name in _includes(os.path.join(ORACLE, "grkan_oracle.c")):
        assert kind == "<" and name in C_LIBRARY_HEADERS, name
    build = open(os.path.join(ORACLE, "oracle.py")).read()
    cmd = re.search(r'cmd = \["gcc",[^\]]*\]', build)
    assert cmd, "gcc command of the oracle build"
    assert "-I" not in cmd.group(0) and "csrc" not in cmd.group(0)


@pytest.mark.parametrize("script, allowed", [
    ("bench.py", ("cpu_baseline", "cpu_baseline_layer", "cpu_baseline_cheby")),
    ("__graft_entry__.py", ("build", "smoke")),
])
def test_product_scripts_import_the_oracle_only_where_allowed(script, allowed):
    path = os.path.join(ROOT, script)
    seen = []
    for mod, level, func in _imports(path):
        if mod.split(".")[0] == "oracle":
            assert func in allowed, (script, mod, func)
            seen.append(func)
    assert seen, f"{script} no longer imports the oracle where expected"
