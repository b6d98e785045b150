"""Build the gfx950 shared library ``libmhc.so`` in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 code
generation switched off (``-target-feature -packed-fp32-ops``), then linked
into one shared library next to this file.  Run ``python -m
birkhoff_projection_amd.build`` or call :func:`build`.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmhc.so")
SOURCES = ["abi.hip", "birkhoff.hip", "birkhoffn.hip", "mix.hip", "layer.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def compile_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libmhc.so``; returns its path."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if out and (verbose or p.returncode != 0):
            print(out, end="", file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
