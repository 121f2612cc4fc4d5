"""The boundary from plain C: tests/c_abi_check.c (C99, -pedantic, warnings
as errors) includes include/sv.h, links libsv.so and calls the host-only
entry points (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "long_context_gqa_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_compiles_as_c_and_host_queries_answer(tmp_path):
    assert os.path.exists(os.path.join(LIBDIR, "libsv.so")), "build the library first"
    exe = tmp_path / "c_abi_check"
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                         os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", str(exe),
                         "-L", LIBDIR, "-lsv", f"-Wl,-rpath,{LIBDIR}"], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "c abi ok" in r.stdout
