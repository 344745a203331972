"""The planners and the host side of the shared helpers under AddressSanitizer
and UndefinedBehaviorSanitizer: tests/plan_fuzz.cpp, built from the
planner's own source with the sanitizers on the host side only, runs 200,000
random argument sets (null, misaligned, overlapping and top-of-address-space
pointers, overflowing sizes, bad element types and paths, batches)."""
from __future__ import annotations

import os
import shutil
import subprocess

from deterministic_collective_movement_amd import build as b

HERE = os.path.dirname(os.path.abspath(__file__))


def test_planners_are_clean_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or os.path.join(b.ROCM, "bin", "hipcc")
    exe = str(tmp_path / "plan_fuzz")
    subprocess.check_call([hipcc, "-x", "hip", "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
                           "-Wno-unused-command-line-argument",
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                           "-Xarch_host", "-fno-sanitize-recover=all",
                           "-I", b.INCLUDE, "-I", b.CSRC, os.path.join(HERE, "plan_fuzz.cpp"),
                           os.path.join(b.CSRC, "rog_plan.cpp"), "-o", exe],
                          stderr=subprocess.DEVNULL)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "200000"], capture_output=True, text=True, timeout=240, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "0 failures" in r.stdout
