"""Build the gfx950 shared library ``libzs.so`` from ``csrc/zs_kernels.hip``
(the kernels) and ``csrc/zs_api.hip`` (the C ABI), and ``libzs_host.so``.

hipcc cross-compiles for gfx950 without a GPU, so this runs anywhere the
ROCm toolchain is installed.  The library is built in-tree, next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
INCLUDE_DIR = os.path.join(REPO_DIR, "include")
SRCS = [os.path.join(PKG_DIR, "csrc", "zs_kernels.hip"),
        os.path.join(PKG_DIR, "csrc", "zs_api.hip")]
# The sources the kernels are compiled from (their hash keys measured traffic).
KERNEL_SRCS = [os.path.join(PKG_DIR, "csrc", "zs_kernels.hip"),
               os.path.join(PKG_DIR, "csrc", "zs_kernels.h")]
LIB = os.path.join(PKG_DIR, "libzs.so")
CEILING_SRC = os.path.join(PKG_DIR, "csrc", "zs_ceiling.hip")
CEILING_LIB = os.path.join(PKG_DIR, "libzs_ceiling.so")
HOST_SRC = os.path.join(PKG_DIR, "csrc", "zs_host.cpp")
HOST_LIB = os.path.join(PKG_DIR, "libzs_host.so")

# Host (ZeRO-Offload) step: OpenMP threads, AVX-512 chosen at run time, no
# contraction and no fast-math so that the results match the device path.
GXX_FLAGS = ["-O3", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
             "-shared", "-Wall"]

ARCH = "gfx950"

# Numerics flags: no fused multiply-add contraction, IEEE divide and square
# root, denormals kept.  Packed fp32 instructions are disabled.
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libzs.so")
    return path


def build_host(verbose: bool = False) -> str:
    """Compile libzs_host.so with g++."""
    tmp = HOST_LIB + ".tmp%d" % os.getpid()
    cmd = ["g++", *GXX_FLAGS, "-I", INCLUDE_DIR, "-o", tmp, HOST_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, HOST_LIB)
    return HOST_LIB


def build_ceiling(verbose: bool = False) -> str:
    """Compile libzs_ceiling.so, the streaming copy bench.py measures beside the
    step (measurement only)."""
    tmp = CEILING_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, CEILING_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


def build(verbose: bool = False) -> str:
    """Compile libzs.so, libzs_host.so and libzs_ceiling.so (always
    recompiles).  Returns the device library path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE_DIR, "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_host(verbose)
    build_ceiling(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
