"""The PEER kernel's cut of a misaligned payload into a byte head, an aligned
16-byte body and a byte tail (split_payload, shared by host and device code),
checked exhaustively on the CPU for every source/destination misalignment:
each output byte is covered exactly once, every aligned source block the body
reads lies inside the payload, and payloads of 48 bytes or more do get a body."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import pytest

from deterministic_collective_movement_amd import build as b

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def split(tmp_path_factory):
    hipcc = shutil.which("hipcc") or os.path.join(b.ROCM, "bin", "hipcc")
    so = str(tmp_path_factory.mktemp("shim") / "libsplit.so")
    subprocess.check_call([hipcc, "-x", "hip", "-O2", "-std=c++17", "-fPIC", "-shared",
                           "--offload-arch=gfx950", "-Wno-unused-command-line-argument",
                           "-I", b.INCLUDE, "-I", b.CSRC, os.path.join(HERE, "split_shim.cpp"), "-o", so],
                          stderr=subprocess.DEVNULL)
    lib = ctypes.CDLL(so)
    lib.rog_test_split.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.POINTER(ctypes.c_uint64)]
    out = (ctypes.c_uint64 * 3)()

    def f(sa, da, S):
        lib.rog_test_split(sa, da, S, out)
        return out[0], out[1], out[2]
    return f


SIZES = list(range(0, 200)) + [255, 256, 257, 4095, 4096, 4097, 65535, 65536, 65537, 262151,
                                (1 << 30) + 7, (1 << 35) + 3]


def check(split, sa, da, S):
    lo, hi, delta = split(sa, da, S)
    assert 0 <= lo <= hi <= S, (sa, da, S, lo, hi)
    assert (hi - lo) % 16 == 0
    if lo == hi:
        assert (lo, hi) == (S, S)        # everything moves as bytes
        assert S < 48, (sa % 16, da % 16, S)
        return
    assert (da + lo) % 16 == 0            # aligned stores
    assert delta == (sa + lo) % 16
    count = (hi - lo) // 16
    if delta == 0:
        first, end = sa + lo, sa + hi     # aligned source vectors, one per output
    else:
        first = sa + lo - delta           # two neighbouring blocks per output
        end = first + 16 * (count + 1)
    assert first % 16 == 0 and end % 16 == 0
    assert sa <= first and end <= sa + S, (sa % 16, da % 16, S, lo, hi, delta)
    assert lo <= 31 and S - hi <= 31      # heads and tails stay short


def test_every_misalignment_and_small_size(split):
    base_s, base_d = 1 << 20, 1 << 32
    for so in range(16):
        for do in range(16):
            for S in SIZES:
                check(split, base_s + so, base_d + do, S)


def test_a_concrete_cut(split):
    # source at 3 mod 16, destination at 9 mod 16: 7 bytes reach the first
    # aligned destination byte, where the source sits 10 bytes into its block;
    # that block starts 3 bytes before the payload, so one more vector moves as
    # bytes and the body starts at byte 23.
    sa, da, S = (1 << 20) + 3, (1 << 24) + 9, 1000
    lo, hi, delta = split(sa, da, S)
    assert (lo, delta) == (23, 10)
    # the body ends where the second source block of its last vector ends
    # inside the payload: 1000 - 23 = 977 bytes -> 61 vectors fit, the last of
    # which would read 16 bytes past the payload's last full block
    assert (hi - lo) // 16 == 60 and S - hi == 17
