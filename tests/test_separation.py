"""The oracle and the product path share no code (no GPU needed): nothing in
oracle/ imports the package or the benchmark, nothing in the package imports
the oracle, the benchmark reaches the oracle only inside its CPU-baseline
leg, and the binding raises when the HIP library is missing instead of
falling back to anything else."""
import ast
import glob
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def imported_modules(path, top_level_only=False):
    """(module name, enclosing function or None) of every import in a file."""
    tree = ast.parse(open(path).read(), filename=path)
    out = []

    def visit(node, func):
        for child in ast.iter_child_nodes(node):
            f = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else func
            if isinstance(child, ast.Import):
                out.extend((a.name, func) for a in child.names)
            elif isinstance(child, ast.ImportFrom) and child.module and child.level == 0:
                out.append((child.module, func))
            visit(child, f)

    visit(tree, None)
    return [(m, f) for m, f in out if not top_level_only or f is None]


def files(pattern):
    return sorted(glob.glob(os.path.join(ROOT, pattern), recursive=True))


@pytest.mark.parametrize("path", files("oracle/*.py"), ids=os.path.basename)
def test_oracle_imports_nothing_of_the_product(path):
    for mod, _ in imported_modules(path):
        assert not mod.startswith(("long_context_gqa_amd", "bench", "__graft_entry__")), (path, mod)


@pytest.mark.parametrize("path", files("long_context_gqa_amd/**/*.py"), ids=os.path.basename)
def test_package_never_imports_the_oracle(path):
    for mod, _ in imported_modules(path):
        assert not mod.startswith("oracle"), (path, mod)


def test_package_sources_name_no_oracle_file():
    for path in files("long_context_gqa_amd/csrc/*") + files("include/*.h"):
        text = open(path, errors="replace").read()
        assert "oracle/" not in text and "#include \"oracle" not in text, path


def test_bench_reaches_the_oracle_only_in_its_cpu_baseline():
    uses = [(m, f) for m, f in imported_modules(os.path.join(ROOT, "bench.py")) if m.startswith("oracle")]
    assert uses and all(f == "cpu_baseline" for _, f in uses), uses


def test_binding_raises_without_the_library(monkeypatch):
    from long_context_gqa_amd import binding as B
    monkeypatch.setattr(B, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libsv.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()
