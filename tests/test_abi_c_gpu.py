"""librog.so from plain C (tests/abi_c_check.c): HIP-runtime allocations and a
stream of its own, no Python or PyTorch in the process; every byte checked
against the C oracle, plus the argument errors and the batched entry point."""
from __future__ import annotations

import os
import subprocess

import pytest

from tests import build_c_check

pytestmark = pytest.mark.gpu


def test_c_consumer_of_the_abi(gpu):
    if not os.path.exists(build_c_check.BIN):
        build_c_check.build_c_check()
    print("running %s" % build_c_check.BIN, flush=True)
    out = subprocess.run([build_c_check.BIN], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "0 failures" in out.stdout
