"""The product path and the oracle stay apart: importing the package (binding
and input generators) loads neither the oracle's Python module nor its
library; no package source imports or links it; the oracle's sources include
nothing of the package; and bench.py and __graft_entry__.py touch the oracle
only inside the CPU baseline, build and smoke functions."""
import ast
import glob
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "recommender_embedding_tables_amd")


@pytest.mark.skipif(not os.path.exists(os.path.join(PKG, "libembtab.so")),
                    reason="the HIP library is not built")
def test_package_import_loads_no_oracle():
    code = ("import sys\n"
            "import recommender_embedding_tables_amd.embtab as eb\n"
            "import recommender_embedding_tables_amd.synth\n"
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]\n"
            "assert not bad, bad\n"
            "maps = open('/proc/self/maps').read()\n"
            "assert 'liboracle' not in maps\n"
            "assert 'libembtab' in maps, 'the HIP library was not loaded'\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr


def test_package_sources_do_not_reference_the_oracle_code():
    pat = re.compile(r"^\s*(import oracle|from oracle\b)|liboracle|oracle/|oracle\.cpp",
                     re.MULTILINE)
    files = (glob.glob(os.path.join(PKG, "*.py")) + glob.glob(os.path.join(PKG, "csrc", "*")) +
             glob.glob(os.path.join(ROOT, "include", "*.h")))
    assert files
    for f in files:
        if f.endswith(".so"):
            continue
        assert not pat.search(open(f, errors="replace").read()), f


def test_oracle_sources_include_nothing_of_the_package():
    for f in glob.glob(os.path.join(ROOT, "oracle", "*.cpp")):
        for line in open(f):
            if line.lstrip().startswith("#include"):
                assert "<" in line, f"{f}: {line.strip()}"  # system headers only
    for f in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        src = open(f).read()
        assert "recommender_embedding_tables_amd" not in src and "embtab" not in src, f


def _oracle_import_sites(path):
    tree = ast.parse(open(path).read())
    sites = []

    def walk(node, fn):
        for child in ast.iter_child_nodes(node):
            name = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else fn
            if isinstance(child, ast.ImportFrom) and (child.module or "").split(".")[0] == "oracle":
                sites.append(fn)
            if isinstance(child, ast.Import) and any(a.name.split(".")[0] == "oracle"
                                                     for a in child.names):
                sites.append(fn)
            walk(child, name)

    walk(tree, None)
    return sites


def test_bench_and_entry_use_the_oracle_only_where_allowed():
    sites = _oracle_import_sites(os.path.join(ROOT, "bench.py"))
    assert sites and set(sites) == {"cpu_baseline"}, sites
    sites = _oracle_import_sites(os.path.join(ROOT, "__graft_entry__.py"))
    assert sites and set(sites) <= {"build", "smoke"}, sites
