"""Build the HIP library in-tree: decode_attention_gqa_amd/libgqa_decode.so.

    python decode_attention_gqa_amd/build.py

Compiles for gfx950 only. Packed fp32 vector instructions are disabled in
device code (`-packed-fp32-ops`); the host pass warns that it does not know
that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "gqa_decode.hip")
LIB = os.path.join(PKG, "libgqa_decode.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False) -> str:
    """Compile the library; returns the path of the shared object."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", os.path.join(PKG, "csrc"), SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


C_SMOKE_SRC = os.path.join(ROOT, "tests", "c_abi", "gqa_c_smoke.c")
C_SMOKE = os.path.join(ROOT, "tests", "c_abi", "gqa_c_smoke")


def build_c_smoke(verbose: bool = False) -> str:
    """Compile the plain-C user of the boundary (tests/c_abi/gqa_c_smoke.c)
    against the built library and the HIP runtime, with gcc: no hipcc, no
    Python, no PyTorch."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", INCLUDE, C_SMOKE_SRC,
           "-L", PKG, "-lgqa_decode", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../decode_attention_gqa_amd", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", C_SMOKE]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed:\n" + r.stdout + r.stderr)
    return C_SMOKE


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_smoke(verbose=True))
