"""The oracle and the GPU path share no code: the oracle's C source includes only C standard
headers, the library's sources include nothing of the oracle, neither side's Python imports the
other, and the seeded input generators (workloads.py) import neither.  Imports are read from
the syntax tree, includes from the preprocessor lines."""
import ast
import os
import re

from conftest import ROOT

C_STD = {"math.h", "stdint.h", "stdlib.h", "string.h", "stddef.h", "stdio.h", "float.h", "limits.h"}


def _includes(path):
    return re.findall(r'^\s*#\s*include\s*[<"]([^>"]+)[>"]', open(path).read(), re.M)


def _imports(path):
    mods = set()
    for node in ast.walk(ast.parse(open(path).read())):
        if isinstance(node, ast.Import):
            mods |= {a.name.split(".")[0] for a in node.names}
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            mods.add(node.module.split(".")[0])
    return mods


def test_oracle_c_includes_only_the_c_library():
    inc = _includes(os.path.join(ROOT, "oracle", "fsdp_oracle.c"))
    assert inc and set(inc) <= C_STD, inc


def test_library_sources_do_not_include_or_import_the_oracle():
    csrc = os.path.join(ROOT, "sharded_fsdp_flatten_amd", "csrc")
    for f in os.listdir(csrc):
        if f.endswith((".hip", ".cpp", ".h")):
            for i in _includes(os.path.join(csrc, f)):
                assert "oracle" not in i, (f, i)
    pkg = os.path.join(ROOT, "sharded_fsdp_flatten_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            assert "oracle" not in _imports(os.path.join(pkg, f)), f


def test_oracle_and_inputs_do_not_import_the_library():
    for path in (os.path.join(ROOT, "oracle", "__init__.py"), os.path.join(ROOT, "workloads.py")):
        mods = _imports(path)
        assert "sharded_fsdp_flatten_amd" not in mods, path
    assert "oracle" not in _imports(os.path.join(ROOT, "workloads.py"))
