"""Build libpostmix.so in-tree with hipcc for gfx950.

    python -m rope_head_mixing_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpostmix.so")
SOURCES = ["postmix_kernels.hip", "postmix_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 instructions stay off: the compiler emits plain fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False, extra_flags=None, out: str | None = None, link_flags=None) -> str:
    """Compile every HIP source and link libpostmix.so next to this file (or
    at `out`, e.g. a checker build with extra host flags)."""
    lib = LIB if out is None else out
    objdir = CSRC if out is None else os.path.dirname(os.path.abspath(out))
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, *(extra_flags or []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *(link_flags or []), "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    for obj in objs:
        os.remove(obj)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
