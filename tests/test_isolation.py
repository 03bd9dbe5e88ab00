"""The oracle and the HIP path stay apart, and the product path has no
fallback.  CPU only (reads sources, loads nothing on a device).

  * nothing under the package imports, links or includes the oracle;
  * the oracle includes nothing of the package (no shared headers, tables or
    helpers);
  * the seeded input generators import neither side;
  * bench.py touches the oracle only inside its cpu_baseline leg;
  * the binding raises when the HIP library is missing instead of computing
    anything itself.
"""
import ast
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "combine_get_dispatch_layout_amd")
ORACLE = os.path.join(ROOT, "oracle")
SRC_EXT = (".py", ".hip", ".hpp", ".cpp", ".h", ".c")


def _sources(top):
    for d, dirs, files in os.walk(top):
        dirs[:] = [x for x in dirs if not x.startswith(("_build", "__pycache__"))]
        for f in files:
            if f.endswith(SRC_EXT):
                yield os.path.join(d, f)


def _code_lines(path):
    """Source lines with comments and docstrings dropped, so a citation of
    the oracle in prose does not count as a use."""
    text = open(path, encoding="utf-8").read()
    if path.endswith(".py"):
        tree = ast.parse(text)
        names = []
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                names += [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                names.append(node.module or "")
            elif isinstance(node, ast.Name):
                names.append(node.id)
            elif isinstance(node, ast.Attribute):
                names.append(node.attr)
            elif isinstance(node, ast.Constant) and isinstance(node.value, str):
                if not _is_docstring(tree, node):
                    names.append(node.value)
        return names
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return [re.sub(r"//.*", "", ln) for ln in text.splitlines()]


def _is_docstring(tree, const):
    for node in ast.walk(tree):
        if isinstance(node, (ast.Module, ast.FunctionDef, ast.ClassDef, ast.AsyncFunctionDef)):
            body = node.body
            if body and isinstance(body[0], ast.Expr) and body[0].value is const:
                return True
    return False


def test_package_never_uses_the_oracle():
    files = list(_sources(PKG))
    assert any(f.endswith("ep.py") for f in files) and any(f.endswith(".hip") for f in files)
    for f in files:
        for ln in _code_lines(f):
            assert "oracle" not in ln.lower(), (f, ln)


def test_oracle_shares_nothing_with_the_package():
    pkg_names = {os.path.basename(f) for f in _sources(PKG)}
    for f in _sources(ORACLE):
        for ln in _code_lines(f):
            assert "combine_get_dispatch_layout_amd" not in ln, (f, ln)
            assert "csrc" not in ln, (f, ln)
            inc = re.match(r'\s*#\s*include\s*[<"]([^>"]+)[>"]', ln) if isinstance(ln, str) else None
            if inc:
                assert os.path.basename(inc.group(1)) not in pkg_names, (f, ln)


def test_input_generators_import_neither_side():
    tree = ast.parse(open(os.path.join(ROOT, "workloads.py"), encoding="utf-8").read())
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods |= {a.name.split(".")[0] for a in node.names}
        elif isinstance(node, ast.ImportFrom):
            mods.add((node.module or "").split(".")[0])
    assert "oracle" not in mods and "combine_get_dispatch_layout_amd" not in mods


def test_bench_uses_the_oracle_only_for_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py"), encoding="utf-8").read())
    uses = []

    def visit(node, fn):
        for child in ast.iter_child_nodes(node):
            name = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else fn
            if isinstance(child, ast.Import) and any(a.name.split(".")[0] == "oracle"
                                                      for a in child.names):
                uses.append(name)
            if isinstance(child, ast.ImportFrom) and (child.module or "").split(".")[0] == "oracle":
                uses.append(name)
            visit(child, name)

    visit(tree, None)
    assert uses and set(uses) == {"cpu_baseline"}


def test_binding_raises_without_the_library(monkeypatch, tmp_path):
    from combine_get_dispatch_layout_amd import ep
    monkeypatch.setattr(ep, "_lib", None)
    monkeypatch.setattr(ep, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        ep.lib()
