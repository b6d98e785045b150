"""AddressSanitizer and UndefinedBehaviorSanitizer over the C ABI's host code.

abi.hip holds every argument check, overlap test, option conversion and
error-string path of the library.  It is compiled here with both sanitizers
on its host code only (device code is unchanged: each -fsanitize flag goes
after -Xarch_host), linked with the library's other objects as build() made
them, and driven by tests/c/abi_from_c.c, compiled by the same clang with the
same sanitizers.  Every call it makes returns before touching a device, so
no GPU is needed; any sanitizer report aborts the run."""
import os
import shutil
import subprocess

import pytest

from birkhoff_projection_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(CLANG), reason="needs the ROCm clang")
def test_c_abi_under_host_sanitizers(tmp_path):
    cc = B.hipcc()
    objs = []
    for src in B.SOURCES:
        if src == "abi.hip":
            continue
        obj = os.path.join(B.BUILD, src.replace(".hip", ".o"))
        assert os.path.exists(obj), "build the library first (__graft_entry__.build())"
        objs.append(obj)
    flags = [f for f in B.compile_flags() if f != "-O3"] + ["-O1", "-g"]
    abi = str(tmp_path / "abi_san.o")
    subprocess.run([cc] + flags + SAN + ["-c", os.path.join(B.CSRC, "abi.hip"), "-o", abi],
                   check=True, capture_output=True, text=True)
    # the host code really is instrumented
    nm = subprocess.run([shutil.which("nm") or "nm", abi], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm
    caller = str(tmp_path / "caller.o")
    subprocess.run([CLANG, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-g",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"),
                    "-c", os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-o", caller],
                   check=True, capture_output=True, text=True)
    exe = str(tmp_path / "abi_san")
    subprocess.run([cc, f"--offload-arch={B.ARCH}", "-fsanitize=address,undefined",
                    "-fno-gpu-sanitize", "-o", exe, caller, abi] + objs,
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
