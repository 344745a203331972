"""Build librog.so (the C-ABI library) in-tree for gfx950.

``build_library()`` compiles the host planner and the HIP kernels (gathers and
rank-ordered sums) with hipcc
for gfx950, then links ``deterministic_collective_movement_amd/librog.so``.
Intermediate objects go to ``_build/`` at the repository root.
``python -m deterministic_collective_movement_amd.build`` does the same.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "librog.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

# Device code: gfx950 only; packed-FP32 instructions disabled.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror",
             "--offload-arch=" + ARCH,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
# Host planner: compiled as HIP source too (it shares the payload-cut helper
# with the kernels), but it holds host code only.
HOST_FLAGS = ["-x", "hip", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror",
              "--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wno-unused-command-line-argument"]


def _run(cmd):
    subprocess.check_call(cmd)


def build_library(out: str = LIB_PATH, defines=(), build_dir: str = BUILD_DIR) -> str:
    """Compile and link librog.so; ``defines`` (e.g. ["ROG_VEC_UNROLL=8"]) go to both compilers."""
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(build_dir, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC, "-I", os.path.join(ROCM, "include")]
    dflags = ["-D" + d for d in defines]
    plan_o = os.path.join(build_dir, "rog_plan.o")
    kern_o = os.path.join(build_dir, "rog_kernels.o")
    red_o = os.path.join(build_dir, "rog_reduce.o")
    _run([hipcc] + HOST_FLAGS + dflags + inc + ["-c", os.path.join(CSRC, "rog_plan.cpp"), "-o", plan_o])
    _run([hipcc] + HIP_FLAGS + dflags + inc + ["-c", os.path.join(CSRC, "rog_kernels.hip"), "-o", kern_o])
    _run([hipcc] + HIP_FLAGS + dflags + inc + ["-c", os.path.join(CSRC, "rog_reduce.hip"), "-o", red_o])
    tmp = out + ".tmp%d" % os.getpid()
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, plan_o, kern_o, red_o,
          "-Wl,-soname,librog.so", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-Wl,--no-undefined", "-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(defines=sys.argv[1:]))
