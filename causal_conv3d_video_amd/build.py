"""Build the HIP library ``libcc3d.so`` in-tree for gfx950.

Compiles the planner (host C++) with g++ and each kernel family and the
launcher with hipcc --offload-arch=gfx950, in parallel, then links one shared
library next to this file.  Run as ``python causal_conv3d_video_amd/build.py``
(not with -m: importing the package loads the library this script builds).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

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

# translation units: (source, compiler)
HIP_SOURCES = (["cc3d_k_g32.hip", "cc3d_k_mfma.hip", "cc3d_k_misc.hip", "cc3d_launch.hip", "cc3d_noalloc.hip",
                "cc3d_k_s1.hip"]
               + ["cc3d_k_few%d.hip" % c for c in range(1, 6)])
CXX_SOURCES = ["cc3d_plan.cpp"]


def _run(cmd):
    print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    if out:
        print(out, flush=True)
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, cmd)


def _objects():
    jobs = []
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        jobs.append((["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC,
                      "-c", os.path.join(CSRC, src), "-o", obj], obj))
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        jobs.append(([HIPCC] + HIP_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    return jobs


def build(verbose=True, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    work = _objects()
    workers = jobs or min(len(work), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda j: _run(j[0]), work))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + [o for _, o in work] + ["-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
