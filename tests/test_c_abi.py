"""The C ABI used from C: tests/c/abi_from_c.c is compiled with gcc -std=c99
-pedantic against include/mhc.h, linked against the built libmhc.so and run.
It calls only paths that return before any device work, so no GPU is needed."""
import os
import shutil
import subprocess

import pytest

from birkhoff_projection_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_caller(tmp_path):
    so = _lib.LIB_PATH
    assert os.path.exists(so), "build the library first (__graft_entry__.build())"
    exe = tmp_path / "abi_from_c"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_from_c.c"),
                    "-o", str(exe), so, "-Wl,-rpath," + os.path.dirname(so)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi ok" in r.stdout
