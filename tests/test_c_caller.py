"""A C program (tests/c_caller.c) compiled with gcc against include/libmoe.h
and linked to libmoe.so: the boundary is plain C (the header compiles as
C99) and a C caller gets the documented sizes and status codes.  No call in
it reaches the GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_moe_layer_gemv_amd")
LIB = os.path.join(PKG, "libmoe.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import runpy
        runpy.run_path(os.path.join(PKG, "_build.py"))["build"]()
    return LIB


def test_header_is_plain_c99():
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-fsyntax-only", "-x", "c", os.path.join(ROOT, "include", "libmoe.h")],
                   check=True)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_calls_the_library(lib, tmp_path):
    exe = tmp_path / "c_caller"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_caller.c"),
                    "-L", PKG, "-l:libmoe.so", f"-Wl,-rpath,{PKG}", "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"
