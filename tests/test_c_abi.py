"""The C ABI from plain C: include/fa.h compiles as C99 (-pedantic -Werror)
and a C program linked against libfa.so gets the documented status codes for
bad arguments, with no GPU (tests/c_abi/abi_check.c)."""
import os
import shutil
import subprocess

import pytest

import io_aware_tiled_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_check.c")

pytestmark = [
    pytest.mark.skipif(not os.path.exists(fa.lib_path()), reason="libfa.so not built"),
    pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available"),
]


def test_c_program_uses_the_abi(tmp_path):
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(fa.lib_path())
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), SRC, fa.lib_path(),
           f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "C ABI checks passed" in r.stdout
