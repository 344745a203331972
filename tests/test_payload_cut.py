"""The PEER kernel's cut of a payload into a byte head, a 16-byte body and a
byte tail (split_payload, shared by host and device code), checked exhaustively
on the CPU for every destination misalignment: each output byte is covered
exactly once, the body starts on a body-alignment boundary of the destination,
heads and tails stay short, and every payload long enough gets a body.  The
body's loads read the source bytes at the body's own payload offsets, so they
lie inside the payload whenever the body lies inside [0, S)."""
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
    """The cut as built, and with the body alignment overridden to 16 .. 256."""
    hipcc = shutil.which("hipcc") or os.path.join(b.ROCM, "bin", "hipcc")
    so = str(tmp_path_factory.mktemp("shim") / "libsplit.so")
    define = [] if request.param is None else ["-DROG_BODY_ALIGN=%d" % request.param]
    subprocess.check_call([hipcc, "-x", "hip", "-O2", "-std=c++17", "-fPIC", "-shared",
                           "--offload-arch=gfx950", "-Wno-unused-command-line-argument"] + define +
                          ["-I", b.INCLUDE, "-I", b.CSRC, os.path.join(HERE, "split_shim.cpp"), "-o", so],
                          stderr=subprocess.DEVNULL)
    lib = ctypes.CDLL(so)
    lib.rog_test_body_align.restype = ctypes.c_uint64
    lib.rog_test_split.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)]
    out = (ctypes.c_uint64 * 2)()

    def f(da, S):
        lib.rog_test_split(da, S, out)
        return out[0], out[1]
    f.align = int(lib.rog_test_body_align())
    return f


SIZES = list(range(0, 400)) + [255, 256, 257, 271, 272, 273, 4095, 4096, 4097, 65535, 65536, 65537,
                                262151, (1 << 30) + 7, (1 << 35) + 3]


def check(split, da, S):
    A = split.align                       # destination alignment of the body
    lo, hi = split(da, S)
    assert 0 <= lo <= hi <= S, (da, S, lo, hi)
    assert (hi - lo) % 16 == 0
    to_line = (-da) % A                   # bytes up to the first A-aligned destination byte
    if lo == hi:
        assert (lo, hi) == (S, S)        # everything moves as bytes
        assert S < to_line + 16, (da % A, S)
        return
    assert (da + lo) % A == 0             # the body starts on a line
    assert lo == to_line                  # ... the first one
    assert S - hi < 16                    # the longest body that fits
    assert lo <= A - 1


def test_every_misalignment_and_small_size(split):
    base_d = 1 << 32
    for do in range(0, 2 * split.align, 1 if split.align <= 16 else 3):
        for S in SIZES:
            check(split, base_d + do, S)


def test_a_concrete_cut(split):
    # destination at 9 mod A: A - 9 bytes reach the first A-aligned byte, and
    # the body runs to the last whole vector of the payload.
    A = split.align
    da, S = (1 << 24) + 9, 5000
    lo, hi = split(da, S)
    assert lo == A - 9
    assert hi == lo + 16 * ((S - lo) // 16)
    assert S - hi < 16


def test_aligned_destination_has_no_head(split):
    lo, hi = split(1 << 40, 4096 + 5)
    assert lo == 0 and hi == 4096


# ---------------------------------------------------------------------------
# XCD-grouped chunk order
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def xcd(tmp_path_factory):
    hipcc = shutil.which("hipcc") or os.path.join(b.ROCM, "bin", "hipcc")
    so = str(tmp_path_factory.mktemp("xcd") / "libxcd.so")
    subprocess.check_call([hipcc, "-x", "hip", "-O2", "-std=c++17", "-fPIC", "-shared",
                           "--offload-arch=gfx950", "-Wno-unused-command-line-argument",
                           "-I", b.INCLUDE, "-I", b.CSRC, os.path.join(HERE, "split_shim.cpp"), "-o", so],
                          stderr=subprocess.DEVNULL)
    lib = ctypes.CDLL(so)
    lib.rog_test_xcd_run.restype = ctypes.c_uint32
    lib.rog_test_xcd_grouped.argtypes = [ctypes.c_uint32, ctypes.c_void_p]

    def f(n):
        import numpy as np
        out = np.empty(max(1, n), np.uint32)
        lib.rog_test_xcd_grouped(n, out.ctypes.data)
        return out[:n]
    f.run = int(lib.rog_test_xcd_run())
    f.lib = lib
    return f


def test_xcd_grouping_is_a_bijection_with_runs(xcd):
    """Every launch size: each chunk is visited exactly once; within whole spans
    of 8 runs, workgroup b (on XCD b mod 8) handles chunks in runs of kXcdRun
    consecutive chunks per XCD; the remainder keeps its order."""
    import numpy as np
    R = xcd.run
    span = 8 * R
    sizes = sorted(set(list(range(0, 3 * span + 9, 7)) + [span - 1, span, span + 1, 5 * span + 3, 65536, 1 << 20]))
    for n in sizes:
        m = xcd(n)
        assert np.array_equal(np.sort(m), np.arange(n, dtype=np.uint32)), n
        full = n - n % span
        b = np.arange(full, dtype=np.int64)
        if full:
            # XCD x = b % 8 works on consecutive chunks x*R + k (mod R) within span b // span
            x, k = b % 8, b // 8
            assert np.array_equal(m[:full], (k // R) * span + x * R + k % R)
        assert np.array_equal(m[full:], np.arange(full, n, dtype=np.uint32)), n


# ---------------------------------------------------------------------------
# The FLAT kernels' chunks (flat_span): shifted so later chunks start on lines
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def flat(xcd):
    lib = xcd.lib
    lib.rog_test_flat_span.argtypes = [ctypes.c_uint32] * 4 + [ctypes.POINTER(ctypes.c_uint32)]
    lib.rog_test_flat_chunk_count.restype = ctypes.c_uint32
    lib.rog_test_flat_chunk_count.argtypes = [ctypes.c_uint32] * 3
    lib.rog_test_flat_shift.restype = ctypes.c_uint32
    lib.rog_test_flat_shift.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    out = (ctypes.c_uint32 * 2)()

    def span(c, chunk, shift, n_vec):
        lib.rog_test_flat_span(c, chunk, shift, n_vec, out)
        return out[0], out[1]
    return span, lib.rog_test_flat_chunk_count, lib.rog_test_flat_shift


def test_flat_chunks_tile_the_output_on_its_lines(flat):
    """Every output size up to 600 vectors, every shift an output address can
    give (0..7) and the chunk lengths of the FLAT kernels (64 and 256 vectors):
    the chunks cover [0, n_vec) exactly once, in order, none empty or longer
    than a chunk, and every chunk after the first starts where the output's
    128-byte lines do (an output at byte 16 * shift past a line)."""
    span, count, _ = flat
    for chunk in (64, 128, 256):
        for shift in range(8):
            for n_vec in range(1, 601):
                nc = count(n_vec, chunk, shift)
                assert nc == -(-(n_vec + shift) // chunk)
                pos = 0
                for c in range(nc):
                    b, n = span(c, chunk, shift, n_vec)
                    assert b == pos and 1 <= n <= chunk, (chunk, shift, n_vec, c, b, n)
                    if c:
                        assert (16 * shift + 16 * b) % 128 == 0
                    pos += n
                assert pos == n_vec, (chunk, shift, n_vec)


def test_flat_chunks_at_the_largest_outputs(flat):
    """Near the top of the 32-bit vector range nothing wraps: shifts up to 7
    below 2^31 vectors, no shift above (the planner's rule), first and last
    chunks exact."""
    span, count, shift_of = flat
    for n_vec, shifts in (((1 << 31) - 1, range(8)), ((1 << 31) - 65, range(8)),
                          ((1 << 32) - 1, [0]), ((1 << 32) - 64, [0]), ((1 << 32) - 65, [0])):
        for shift in shifts:
            nc = count(n_vec, 64, shift)
            assert nc == -(-(n_vec + shift) // 64)
            assert span(0, 64, shift, n_vec) == (0, 64 - shift)
            b, n = span(nc - 1, 64, shift, n_vec)
            assert b + n == n_vec and 1 <= n <= 64 and b == (nc - 1) * 64 - shift
    assert shift_of((1 << 34) + 16 * 5, (1 << 31) - 1) == 5
    assert shift_of((1 << 34) + 16 * 5, 1 << 31) == 0
    assert [shift_of((1 << 34) + 16 * k, 1000) for k in range(16)] == [k % 8 for k in range(16)]


# ---------------------------------------------------------------------------
# Byte-window cut of the PEER body (misaligned sources)
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def cut16(tmp_path_factory):
    hipcc = shutil.which("hipcc") or os.path.join(b.ROCM, "bin", "hipcc")
    so = str(tmp_path_factory.mktemp("cut16") / "libcut16.so")
    subprocess.check_call([hipcc, "-x", "hip", "-O2", "-std=c++17", "-fPIC", "-shared",
                           "--offload-arch=gfx950", "-Wno-unused-command-line-argument",
                           "-I", b.INCLUDE, "-I", b.CSRC, os.path.join(HERE, "split_shim.cpp"), "-o", so],
                          stderr=subprocess.DEVNULL)
    lib = ctypes.CDLL(so)
    lib.rog_test_cut16.argtypes = [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_uint32, ctypes.c_void_p]
    out = ctypes.create_string_buffer(16)

    def f(window, m):
        lib.rog_test_cut16(bytes(window[:16]), bytes(window[16:]), m, out)
        return out.raw
    f.shift = int(lib.rog_test_peer_shift())
    return f


def test_cut16_takes_bytes_m_to_m_plus_16(cut16):
    """For every shift m the cut returns bytes [m, m + 16) of the 32-byte pair:
    the unaligned payload bytes a lane stores, rebuilt from two aligned granules."""
    import random
    rng = random.Random(7)
    for m in range(16):
        for _ in range(50):
            w = bytes(rng.randrange(256) for _ in range(32))
            assert cut16(w, m) == w[m:m + 16], m
        # distinct bytes: a swapped or repeated dword would show
        w = bytes(range(32))
        assert cut16(w, m) == w[m:m + 16], m


def test_peer_shift_mode_is_a_known_one(cut16):
    assert cut16.shift in (0, 1, 2)


# ---------------------------------------------------------------------------
# The sum's granule-form cut, anchored on source 0's 128-byte lines
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def anchored(tmp_path_factory):
    hipcc = shutil.which("hipcc") or os.path.join(b.ROCM, "bin", "hipcc")
    so = str(tmp_path_factory.mktemp("anch") / "libanch.so")
    subprocess.check_call([hipcc, "-x", "hip", "-O2", "-std=c++17", "-fPIC", "-shared",
                           "--offload-arch=gfx950", "-Wno-unused-command-line-argument",
                           "-I", b.INCLUDE, "-I", b.CSRC, os.path.join(HERE, "split_shim.cpp"), "-o", so],
                          stderr=subprocess.DEVNULL)
    lib = ctypes.CDLL(so)
    lib.rog_test_split_anchored.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                            ctypes.POINTER(ctypes.c_uint64)]
    out = (ctypes.c_uint64 * 2)()

    def f(da, S, anchor):
        lib.rog_test_split_anchored(da, S, anchor, out)
        return out[0], out[1]
    return f


def test_split_anchored_every_alignment(anchored):
    """For every output and anchor alignment (mod 256, in 2-byte steps as for
    2-byte elements) and sizes around the body's start: the body starts at the
    smallest offset where the output is 16-byte aligned and the anchor's granule
    run starts a 128-byte line, holds whole 16-byte vectors, and leaves a tail
    under 16 bytes; sizes too small for a body leave it empty."""
    base = 1 << 40
    for do in range(0, 256, 2):
        for ao in range(0, 256, 2):
            want_lo = next(l for l in range(0, 256) if (do + l) % 16 == 0 and (ao + l) % 128 < 16)
            assert want_lo < 128
            for S in (0, 1, want_lo + 14, want_lo + 15, want_lo + 16, want_lo + 17, 1000, 4096 + 7):
                lo, hi = anchored(base + do, S, base + 512 + ao)
                if S < want_lo + 16:
                    assert (lo, hi) == (S, S), (do, ao, S)
                    continue
                assert lo == want_lo, (do, ao, S, lo)
                assert (hi - lo) % 16 == 0 and hi <= S and S - hi < 16, (do, ao, S, lo, hi)
