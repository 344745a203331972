"""Device-code resources of every kernel, from the gfx950 assembly that hipcc
emits here on the CPU: no kernel may spill to scratch or use a dynamic stack
(a streaming copy has nothing to spill; a spill means an address or unroll
regression), and each stays within the VGPR budget of its workgroup size."""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from deterministic_collective_movement_amd import build as b


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    hipcc = shutil.which("hipcc") or os.path.join(b.ROCM, "bin", "hipcc")
    ks = {}
    for src in ("rog_kernels.hip", "rog_reduce.hip"):
        out = str(tmp_path_factory.mktemp("asm") / (src + ".s"))
        subprocess.check_call([hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "--offload-device-only",
                               "-S", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "-Wno-unused-command-line-argument", "-I", b.INCLUDE, "-I", b.CSRC,
                               os.path.join(b.CSRC, src), "-o", out],
                              stderr=subprocess.DEVNULL)
        ks.update(_parse(open(out).read()))
    return ks


def _parse(text):
    meta = text[text.index("amdhsa.kernels:"):]
    ks = {}
    for block in re.split(r"\n  - \.", meta)[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        get = lambda k: int(re.search(r"\.%s:\s+(\d+)" % k, block).group(1))  # noqa: E731
        explicit = [(int(o), int(z)) for o, z, kind in
                    re.findall(r"\.offset:\s+(\d+)\s+\.size:\s+(\d+)\s+\.value_kind:\s+(\w+)", block)
                    if not kind.startswith("hidden_")]
        ks[name.group(1)] = {"scratch": get("private_segment_fixed_size"), "vgpr": get("vgpr_count"),
                             "max_wg": get("max_flat_workgroup_size"), "explicit_args": explicit,
                             "dyn_stack": re.search(r"uses_dynamic_stack:\s+true", block) is not None}
    return ks


def test_every_kernel_is_present(kernels):
    names = " ".join(kernels)
    for k in ("rog_flat_kernel", "rog_flat_single_kernel", "rog_peer_kernel", "rog_peer_single_kernel",
              "rog_batch_kernel", "rog_reduce_kernel", "rog_reduce_single_kernel"):
        assert k in names, k
    assert len(kernels) >= 18


def test_no_scratch_and_vgprs_fit(kernels):
    for name, k in kernels.items():
        assert k["scratch"] == 0, (name, k)
        assert not k["dyn_stack"], name
        # 512 VGPRs per SIMD lane slot; a workgroup of w threads puts w/256
        # waves on each of the 4 SIMDs of a CU.
        budget = 512 // max(1, k["max_wg"] // 256)
        assert k["vgpr"] <= min(budget, 512), (name, k)


def test_one_argument_struct_at_offset_zero(kernels):
    """The multi-WG kernels read their argument struct through the
    kernel-argument segment pointer, as the struct at offset 0: every kernel
    takes exactly one explicit argument, by value, at offset 0."""
    for name, k in kernels.items():
        assert len(k["explicit_args"]) == 1, (name, k["explicit_args"])
        assert k["explicit_args"][0][0] == 0, (name, k["explicit_args"])
