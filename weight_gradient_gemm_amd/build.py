"""Builds libforge.so in-tree for gfx950.

    python -m weight_gradient_gemm_amd.build

The host-only validation is compiled with g++; the HIP translation unit with
hipcc. Floating-point flags are pinned: no contraction of multiply-add pairs
(the optimizer arithmetic is rounded exactly as written), IEEE-rounded float32
division and square root, and no packed-fp32 instructions.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libforge.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra"]


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libforge.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


# HIP translation units (compiled in parallel) and the host-only validation.
HIP_UNITS = ("host.hip", "forge.hip", "forge_dgrad.hip", "forge_fp8.hip")


def build(verbose: bool = True) -> str:
    """Compile every source and link libforge.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    v_obj = os.path.join(BUILD, "validate.o")
    jobs = [["g++", *CXX_FLAGS, *inc, "-c", os.path.join(CSRC, "validate.cpp"), "-o", v_obj]]
    objs = [v_obj]
    for unit in HIP_UNITS:
        obj = os.path.join(BUILD, unit.replace(".hip", ".o"))
        jobs.append([_hipcc(), *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, unit), "-o", obj])
        objs.append(obj)
    procs = []
    for cmd in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
    failed = [cmd for cmd, pr in zip(jobs, procs) if pr.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    tmp = LIB + ".tmp"
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
