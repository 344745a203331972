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


@pytest.fixture(scope="module", params=[None, 16, 64, 128, 256], ids=["built", "A16", "A64", "A128", "A256"])
def split(request, tmp_path_factory):
    """The cut as built, and with the body alignment overridden to 16, 128, 256."""
    hipcc = shutil.which("hipcc") or os.path.join(b.ROCM, "bin", "hipcc")
    so = str(tmp_path_factory.mktemp("shim") / "libsplit.so")
    define = [] if request.param is None else ["-DROG_BODY_ALIGN=%d" % request.param]
    subprocess.check_call([hipcc, "-x", "hip", "-O2", "-std=c++17", "-fPIC", "-shared",
                           "--offload-arch=gfx950", "-Wno-unused-command-line-argument"] + define +
                          ["-I", b.INCLUDE, "-I", b.CSRC, os.path.join(HERE, "split_shim.cpp"), "-o", so],
                          stderr=subprocess.DEVNULL)
    lib = ctypes.CDLL(so)
    lib.rog_test_body_align.restype = ctypes.c_uint64
    lib.rog_test_split.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.POINTER(ctypes.c_uint64)]
    out = (ctypes.c_uint64 * 3)()

    def f(sa, da, S):
        lib.rog_test_split(sa, da, S, out)
        return out[0], out[1], out[2]
    f.align = int(lib.rog_test_body_align())
    return f


SIZES = list(range(0, 400)) + [255, 256, 257, 4095, 4096, 4097, 65535, 65536, 65537, 262151,
                                (1 << 30) + 7, (1 << 35) + 3]


def check(split, sa, da, S):
    A = split.align                       # destination alignment of the body
    lo, hi, delta = split(sa, da, S)
    assert 0 <= lo <= hi <= S, (sa, da, S, lo, hi)
    assert (hi - lo) % 16 == 0
    if lo == hi:
        assert (lo, hi) == (S, S)        # everything moves as bytes
        assert S < A + 48, (sa % 16, da % 16, S)
        return
    assert (da + lo) % 16 == 0            # aligned stores
    assert (da + lo) % A == 0 or (da + lo) % A == 16   # the body starts on (or one vector past) a line
    assert delta == (sa + lo) % 16
    count = (hi - lo) // 16
    if delta == 0:
        first, end = sa + lo, sa + hi     # aligned source vectors, one per output
    else:
        first = sa + lo - delta           # two neighbouring blocks per output
        end = first + 16 * (count + 1)
    assert first % 16 == 0 and end % 16 == 0
    assert sa <= first and end <= sa + S, (sa % 16, da % 16, S, lo, hi, delta)
    assert lo <= A + 15 and S - hi <= 31  # heads and tails stay short


def test_every_misalignment_and_small_size(split):
    base_s, base_d = 1 << 20, 1 << 32
    for so in range(16):
        for do in range(0, 2 * split.align, 1 if split.align <= 16 else 3):
            for S in SIZES:
                check(split, base_s + so, base_d + do, S)


def test_a_concrete_cut(split):
    # source at 3 mod 16, destination at 9 mod A: A - 9 bytes reach the first
    # A-aligned destination byte, where the source sits (3 + A - 9) mod 16 bytes
    # into its block.
    A = split.align
    sa, da, S = (1 << 20) + 3, (1 << 24) + 9, 5000
    lo, hi, delta = split(sa, da, S)
    h = A - 9
    d = (3 + h) % 16
    want_lo = h + (16 if d > h else 0)    # the first block would start before the payload
    assert (lo, delta) == (want_lo, (3 + want_lo) % 16)
    # the last body vector's second source block ends inside the payload
    assert sa + lo - delta + 16 * ((hi - lo) // 16 + 1) <= sa + S
    assert S - hi <= 31
