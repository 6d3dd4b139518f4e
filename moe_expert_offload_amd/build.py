"""Builds libmoe.so (HIP kernels for gfx950 + host orchestrator + C ABI) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fno-gpu-flush-denormals-to-zero",
    # packed FP32 instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


CXX = os.environ.get("CXX", "g++")
# host-only C++ (no device code); vector paths are selected at run time per function
CXXFLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(HERE, "csrc")]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def host_sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.cpp")))


def build(verbose: bool = False) -> str:
    srcs = sources()
    objs = []
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    for s in srcs:
        o = os.path.join(HERE, "_build", os.path.basename(s) + ".o")
        cmd = [HIPCC, *FLAGS, "-c", s, "-o", o]
        cmd.remove("-shared")
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(o)
    for s in host_sources():
        o = os.path.join(HERE, "_build", os.path.basename(s) + ".o")
        cmd = [CXX, *CXXFLAGS, "-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(o)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp, "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
