"""Build the HIP library libdspark_ctx_kv.so in-tree with hipcc for gfx950.

Usage: python -m speculative_decoding_draft_02_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdspark_ctx_kv.so")
SOURCES = ["ctx_kv_kernel.hip", "ctx_kv_writer.cpp", "qknorm_insert_kernel.hip", "qknorm_insert.cpp",
           "project_kernel.hip", "project.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the DSpark context-KV library needs ROCm's hipcc")


def command(out: str) -> list:
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-command-line-argument",
            # packed fp32 ops stay off: the compiler must not form v_pk_* f32 math
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]\
        + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out]


def build(verbose: bool = False) -> str:
    """Compile every source into LIB (always recompiles) and return its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
