"""Build libpkv.so for gfx950 with hipcc (in-tree, next to the binding).

    python paged_kv_cache_13_amd/csrc/build.py

Compiles every .hip source here into one shared library.  Packed fp32 VALU
ops are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
SOURCES = ["decode.hip", "scatter.hip", "abi.hip", "alloc.hip"]
OUT = os.path.join(PKG, "libpkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", HERE,
]


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + [os.path.join(HERE, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd, cwd=HERE)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
