"""Build libddtree.so in-tree with hipcc for gfx950.

    python -m block_diffusion_draft_ddtree_amd.build_lib

All HIP sources under csrc/ are compiled and linked into one shared library
next to this file. Packed fp32 ops are disabled for the device code.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libddtree.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libddtree)")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [
        hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
        *sources(), "-o", tmp,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


C_DRIVER_SRC = os.path.join(ROOT, "tests", "c", "abi_round.c")
C_DRIVER = os.path.join(ROOT, "tests", "c", "abi_round")


def build_c_driver(verbose: bool = False) -> str:
    """Compile the plain-C program that runs a round through the C ABI
    (host code only: gcc against the HIP runtime and libddtree)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = [
        shutil.which("gcc") or "gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
        "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
        C_DRIVER_SRC, "-o", C_DRIVER + ".tmp", "-L", PKG, "-lddtree",
        "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
        "-Wl,-rpath,$ORIGIN/../../block_diffusion_draft_ddtree_amd",
        "-Wl,-rpath," + os.path.join(rocm, "lib"),
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(C_DRIVER + ".tmp", C_DRIVER)
    return C_DRIVER


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_driver(verbose=True))
