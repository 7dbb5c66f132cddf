"""Ahead-of-time build of libmoeperm.so for gfx950 (MI355X).

Each HIP source is compiled with hipcc for gfx950 only and the objects are
linked into one shared library next to this file.  Run it as a script
(``python unpermute_moe_make_amd/build.py``) -- importing the package needs the
library it builds -- or call :func:`build` after loading this file by path.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoeperm.so")
SOURCES = ["api.hip", "row_map.hip", "permute.hip", "chunks.hip", "router.hip", "mask.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # Plain fp32 arithmetic only: no implicit contraction, no fast-math, and
    # no packed-fp32 instructions (the kernels write explicit fmaf where the
    # method fuses).
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libmoeperm.so; returns its path."""
    objdir = tempfile.mkdtemp(prefix="moeperm_build_")
    try:
        objs = []
        for src in SOURCES:
            obj = os.path.join(objdir, src.replace(".hip", ".o"))
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd)
            objs.append(obj)
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
