"""Build tests/abi_c_check.c (a plain C consumer of librog.so, checked against
the C oracle) into _build/abi_c_check.  Called by __graft_entry__.build()."""
from __future__ import annotations

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
PKG_DIR = os.path.join(ROOT, "deterministic_collective_movement_amd")
BIN = os.path.join(ROOT, "_build", "abi_c_check")


def build_c_check() -> str:
    os.makedirs(os.path.dirname(BIN), exist_ok=True)
    tmp = BIN + ".tmp%d" % os.getpid()
    subprocess.check_call([
        "gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
        os.path.join(ROOT, "tests", "abi_c_check.c"), os.path.join(ROOT, "oracle", "rog_oracle.c"),
        os.path.join(PKG_DIR, "librog.so"), "-Wl,-rpath,$ORIGIN/../deterministic_collective_movement_amd",
        "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
        "-o", tmp])
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build_c_check())
