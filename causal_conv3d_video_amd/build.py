"""Build the HIP library ``libcc3d.so`` in-tree for gfx950.

Compiles the planner (host C++) with g++ and the kernels and launcher with
hipcc --offload-arch=gfx950, then links one shared library next to this file.
Run as ``python causal_conv3d_video_amd/build.py`` (not with -m: importing
the package loads the library this script builds).
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcc3d.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 arithmetic is disabled for every HIP file (ordinary scalar fp32
# code only).
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    plan_o = os.path.join(BUILD, "cc3d_plan.o")
    fwd_o = os.path.join(BUILD, "cc3d_forward.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC,
          "-c", os.path.join(CSRC, "cc3d_plan.cpp"), "-o", plan_o])
    _run([HIPCC] + HIP_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "cc3d_forward.hip"),
                                "-o", fwd_o])
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", plan_o, fwd_o, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
