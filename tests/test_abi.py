"""The C ABI on the CPU: exported symbols, constants, validation, dispatch and
grid sizing (include/rog.h).  No test here launches a kernel: rog_plan never
calls HIP, and every call of rog_gather / rog_gather_many below fails
validation (or has nothing to copy) before any HIP call."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from deterministic_collective_movement_amd import rog

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rog.h")

A = 1 << 20          # a 16-byte aligned fake device address
FLAT_BLOCK, FLAT_UNROLL = 64, 1      # multi-WG FLAT: threads per WG, vectors per lane per chunk
SINGLE_UNROLL = 4                    # single-WG FLAT: vectors per lane per chunk
SINGLE_PEER_UNROLL = 4               # single-WG PEER: 16-byte vectors per thread
PEER_BLOCK = 64                      # multi-WG PEER: one wave per workgroup, 64 body vectors each
GATHER_NT_LOAD_MIN_BYTES = 128 << 20   # source bytes from which a single gather's loads are non-temporal
OK, INVALID, OVERLAP, TOO_LARGE = (rog.ROG_OK, rog.ROG_ERR_INVALID_ARGUMENT,
                                   rog.ROG_ERR_OVERLAP, rog.ROG_ERR_TOO_LARGE)


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"ROG_API\s+[\w\s\*]+?\b(rog_\w+)\s*\(", text)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"rog_gather", "rog_gather_ex", "rog_gather_many", "rog_plan",
            "rog_single_wg_max_bytes", "rog_max_peers", "rog_max_batch",
            "rog_max_batch_pointers", "rog_last_hip_error", "rog_status_string"} <= names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(rog.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.check_output(["nm", "-D", "--defined-only", rog.library_path()]).decode()
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name


def test_library_links_one_hip_runtime():
    out = subprocess.check_output(["readelf", "-d", rog.library_path()]).decode()
    needed = re.findall(r"\(NEEDED\).*\[(.*)\]", out)
    assert sum(n.startswith("libamdhip64") for n in needed) == 1
    assert "libtorch" not in " ".join(needed)


def test_constants():
    assert rog.rog_max_peers() >= 8          # the pages' groups have up to eight ranks
    assert rog.rog_max_batch() >= 16
    assert rog.rog_max_batch_pointers() >= 16 * 4
    assert rog.rog_single_wg_max_bytes() > 0
    assert rog.rog_last_hip_error() == 0
    assert rog.rog_status_string(0) == "ROG_OK"
    assert rog.rog_status_string(4) == "ROG_ERR_LAUNCH"
    assert rog.rog_status_string(99) == "ROG_ERR_UNKNOWN"


# ---------------------------------------------------------------------------
# Validation (every code path returns before any HIP call)
# ---------------------------------------------------------------------------

def st(srcs, S, out, path=rog.ROG_PATH_AUTO, W=None):
    return rog.rog_status_of_ptrs(srcs, len(srcs) if W is None else W, S, out, path)


def test_invalid_arguments():
    assert st(None, 16, A, W=2) == INVALID                # srcs array NULL
    assert st([A], 16, A + 4096, W=0) == INVALID          # W < 1
    M = rog.rog_max_peers()
    assert st([A + 64 * i for i in range(M + 1)], 16, 2 * A) == INVALID
    assert st([A + 64 * i for i in range(M)], 16, 2 * A) == OK
    assert st([A, 0], 16, 2 * A) == INVALID               # a NULL payload
    assert st([A, A + 64], 16, 0) == INVALID              # NULL output
    assert st([A], 16, 2 * A, path=7) == INVALID          # unknown path
    assert st([A], 16, 2 * A, path=-1) == INVALID
    info_null = rog.lib().rog_plan(rog._ptr_array([A]), 1, 16, ctypes.c_void_p(2 * A), 0, None)
    assert info_null == INVALID


def test_zero_bytes_is_a_no_op_even_with_null_pointers():
    assert st([0, 0], 0, 0) == OK
    p = rog.rog_plan_ptrs([0, 0, 0], 0, 0)
    assert p["kernel"] == "none" and p["grid"] == 0
    # rog_gather with S == 0 enqueues nothing (no HIP call), so it succeeds here.
    rog.rog_gather_ptrs([0, 0], 0, 0)
    rog.rog_gather_many_ptrs([[0, 0], [0, 0]], [0, 0], [0, 0], 2)
    rog.rog_gather_many_ptrs([], [], [], 3)


def test_too_large():
    big = (1 << 64) - 1
    assert st([A, A], big // 2 + 1, 3 * A) == TOO_LARGE   # W*S overflows
    assert st([A], 1 << 36, 1 << 40) == TOO_LARGE         # 2^36 bytes = 2^32 vectors
    assert st([A], (1 << 36) - 16, 1 << 40) == OK
    assert st([A, A], 1 << 35, 1 << 40) == TOO_LARGE


def test_address_wrap_is_invalid():
    top = (1 << 64) - 64
    assert st([top], 128, A) == INVALID
    assert st([A], 128, top) == INVALID


def test_overlap_rules():
    S = 256
    out = 1 << 24
    # a source partially inside the output
    assert st([A, out + 10], S, out) == OVERLAP
    # a source covering the output start
    assert st([out - 100, A], S, out) == OVERLAP
    # exact in place: payload r already in segment r
    assert st([A, out + S, A + 4096], S, out) == OK
    assert st([out, A], S, out) == OK
    # a payload sitting in another rank's segment races with that segment's copy
    assert st([out + S, A], S, out) == OVERLAP
    # touching ranges do not overlap
    assert st([out - S, out + 2 * S], S, out) == OK
    # aliased sources are fine
    assert st([A, A, A], S, out) == OK


def test_validation_errors_from_rog_gather_before_any_launch():
    with pytest.raises(rog.RogArgumentError) as e:
        rog.rog_gather_ptrs([A, A + 8], 16, A + 4)
    assert e.value.status == OVERLAP
    with pytest.raises(rog.RogArgumentError) as e:
        rog.rog_gather_ptrs([A, 0], 16, 2 * A)
    assert e.value.status == INVALID
    with pytest.raises(rog.RogArgumentError):
        rog.rog_gather_ptrs([A], 1 << 36, 1 << 40)


def test_batch_validation():
    W = 4
    n_max = rog.rog_max_batch()
    srcs = [[A + 4096 * (t * W + r) for r in range(W)] for t in range(n_max + 1)]
    outs = [1 << 30 | (t << 20) for t in range(n_max + 1)]
    with pytest.raises(rog.RogArgumentError) as e:
        rog.rog_gather_many_ptrs(srcs, [64] * (n_max + 1), outs, W)
    assert e.value.status == TOO_LARGE
    # n * W above the pointer capacity
    Wp = rog.rog_max_batch_pointers() // 4 + 1
    with pytest.raises(rog.RogArgumentError) as e:
        rog.rog_gather_many_ptrs([[A] * Wp] * 4, [16] * 4, [1 << 30 | (t << 24) for t in range(4)], Wp)
    assert e.value.status == TOO_LARGE
    # two outputs overlap
    with pytest.raises(rog.RogArgumentError) as e:
        rog.rog_gather_many_ptrs([[A] * 2, [A] * 2], [64, 64], [1 << 30, (1 << 30) + 100], 2)
    assert e.value.status == OVERLAP
    # a source of tensor 1 lies in tensor 0's output
    with pytest.raises(rog.RogArgumentError) as e:
        rog.rog_gather_many_ptrs([[A] * 2, [(1 << 30) + 8, A]], [64, 64], [1 << 30, 1 << 31], 2)
    assert e.value.status == OVERLAP
    # a NULL payload in the second tensor
    with pytest.raises(rog.RogArgumentError) as e:
        rog.rog_gather_many_ptrs([[A] * 2, [0, A]], [64, 64], [1 << 30, 1 << 31], 2)
    assert e.value.status == INVALID
    # W out of range, negative n
    assert rog.lib().rog_gather_many(None, 0, 0, None) == INVALID
    assert rog.lib().rog_gather_many(None, -1, 2, None) == INVALID
    assert rog.lib().rog_gather_many(None, 2, 2, None) == INVALID


# ---------------------------------------------------------------------------
# Classification, dispatch, grid
# ---------------------------------------------------------------------------

def test_flat_iff_output_size_and_every_payload_aligned():
    S = 4096
    out = 1 << 24
    assert rog.rog_plan_ptrs([A, A + S], S, out)["kernel"] == "flat"
    assert rog.rog_plan_ptrs([A, A + S + 1], S, out)["kernel"] == "peer"
    assert rog.rog_plan_ptrs([A, A + S], S, out + 8)["kernel"] == "peer"
    assert rog.rog_plan_ptrs([A, A + 4 * S], S + 8, out)["kernel"] == "peer"
    for off in range(1, 16):
        assert rog.rog_plan_ptrs([A + off], S, out)["kernel"] == "peer"


def test_vec_ok_mask_per_peer():
    # S % 16 == 8: segment r starts at out + 8r, so only even ranks are aligned
    # on the destination side; sources alternate aligned / misaligned by 3.
    S = 8 + 16 * 10
    out = 1 << 24
    srcs = [A + 4096 * r + (0 if r % 4 < 2 else 3) for r in range(8)]
    p = rog.rog_plan_ptrs(srcs, S, out, rog.ROG_PATH_MULTI_WG)
    want = 0
    for r in range(8):
        if (srcs[r] % 16 == 0) and ((out + r * S) % 16 == 0):
            want |= 1 << r
    assert p["kernel"] == "peer"
    assert p["vec_ok_mask"] == want == 0b00010001  # ranks 0 and 4
    assert p["units"] == 8 * S


def test_auto_path_follows_the_exported_crossover_inclusively():
    X = rog.rog_single_wg_max_bytes()
    out = 1 << 30
    for W in (1, 2, 4, 8):
        if X % W:
            continue
        S = X // W
        srcs = [A + (S + 4096) * r for r in range(W)]
        assert rog.rog_plan_ptrs(srcs, S, out)["path"] == "single_wg"
        srcs = [A + (S + 4096 + 16) * r for r in range(W)]
        assert rog.rog_plan_ptrs(srcs, S + 1, out)["path"] == "multi_wg"
    # forced paths are honoured either side of the crossover
    assert rog.rog_plan_ptrs([A], 1 << 20, out, rog.ROG_PATH_SINGLE_WG)["path"] == "single_wg"
    assert rog.rog_plan_ptrs([A], 16, out, rog.ROG_PATH_MULTI_WG)["path"] == "multi_wg"


def test_grid_sizes():
    out = 1 << 34
    # FLAT multi-WG: one wave per chunk of 64*U vectors.
    for W, S in [(2, 1024), (8, 1 << 20), (8, 64 << 20), (3, 16 * 257), (1, 16)]:
        srcs = [A + (S + 4096) * r for r in range(W)]
        p = rog.rog_plan_ptrs(srcs, S, out, rog.ROG_PATH_MULTI_WG)
        n_vec = W * S // 16
        chunks = -(-n_vec // (64 * FLAT_UNROLL))
        assert p["kernel"] == "flat" and p["block"] == FLAT_BLOCK
        assert p["grid"] == max(1, -(-chunks // (FLAT_BLOCK // 64)))
        # an output 16 * k bytes past a 128-byte line: the first chunk is k
        # vectors short, so one more chunk may be needed
        for k in range(8):
            q = rog.rog_plan_ptrs(srcs, S, out + 16 * k, rog.ROG_PATH_MULTI_WG)
            assert q["kernel"] == "flat" and q["grid"] == max(1, -(-(n_vec + k) // (64 * FLAT_UNROLL))), (W, S, k)
        s = rog.rog_plan_ptrs(srcs, S, out, rog.ROG_PATH_SINGLE_WG)
        # 1 KiB wave chunks while 16 waves cover the output, 4 KiB beyond
        u = 1 if n_vec <= 1024 else SINGLE_UNROLL
        single_chunks = -(-n_vec // (64 * u))
        assert s["grid"] == 1 and s["block"] == min(1024, max(64, 64 * single_chunks))
    # PEER multi-WG: W payloads, each cut into 1 KiB body chunks (enough for
    # the longest possible body, S // 16 vectors), one wave per chunk.
    for W, S in [(4, 100_001), (2, 1), (8, 1023), (3, 64 * 16 * 7 + 15)]:
        srcs = [A + 1 + (S + 4096) * r for r in range(W)]
        p = rog.rog_plan_ptrs(srcs, S, out, rog.ROG_PATH_MULTI_WG)
        assert p["kernel"] == "peer" and p["vec_ok_mask"] == 0 and p["block"] == PEER_BLOCK
        assert p["grid"] == W * max(1, -(-(S // 16) // 64)), (W, S)


def test_single_wg_peer_block_fits_the_largest_payload():
    out = 1 << 34
    # (W, S, source offset, output offset)
    for W, S, io, oo in [(2, 1, 1, 1), (2, 4095, 1, 1), (1, 16 * 5000 + 3, 0, 0), (2, 1 << 20, 3, 1)]:
        p = rog.rog_plan_ptrs([A + io + (S + 4096) * r for r in range(W)], S, out + oo,
                              rog.ROG_PATH_SINGLE_WG)
        assert p["kernel"] == "peer" and p["grid"] == 1 and p["units"] == W * S
        want_threads = -(-(S // 16) // SINGLE_PEER_UNROLL)
        assert p["block"] == min(1024, max(64, -(-want_threads // 64) * 64)), S


def test_grid_times_block_fits_a_dispatch():
    """An AMD dispatch counts work-items in 32 bits: grid * block < 2^32 even at
    the largest output (the kernels grid-stride over what a capped grid leaves)."""
    S = ((1 << 36) - 16) // 8 // 16 * 16
    p = rog.rog_plan_ptrs([A + (S + 4096) * r for r in range(8)], S, 1 << 45, rog.ROG_PATH_MULTI_WG)
    assert p["kernel"] == "flat"
    assert p["grid"] * p["block"] < (1 << 32)
    p = rog.rog_plan_ptrs([A + 1 + (S + 4096) * r for r in range(8)], S, 1 << 45, rog.ROG_PATH_MULTI_WG)
    assert p["kernel"] == "peer"
    assert p["grid"] * p["block"] < (1 << 32)


def test_nt_load_policy_follows_source_bytes():
    out = 1 << 40
    # FLAT (everything 16-byte aligned)
    for W, S, want in [(8, 64 << 20, True), (8, 16 << 20, True), (8, 8 << 20, False),
                       (1, GATHER_NT_LOAD_MIN_BYTES, True), (1, GATHER_NT_LOAD_MIN_BYTES - 16, False),
                       (2, 1024, False)]:
        srcs = [A + (S + 4096) * r for r in range(W)]
        p = rog.rog_plan_ptrs(srcs, S, out)
        assert p["kernel"] == "flat" and p["nt_loads"] is want, (W, S)
    # PEER (sources one byte off)
    for W, S, want in [(8, 64 << 20, True), (8, 16 << 20, True), (8, (16 << 20) - 1, False),
                       (1, GATHER_NT_LOAD_MIN_BYTES, True), (1, GATHER_NT_LOAD_MIN_BYTES - 16, False),
                       (8, 8 << 20, False)]:
        srcs = [A + 1 + (S + 4096) * r for r in range(W)]
        p = rog.rog_plan_ptrs(srcs, S, out)
        assert p["kernel"] == "peer" and p["nt_loads"] is want, (W, S)


def _divide(v, magic, sh1, sh2):
    t = (v * magic) >> 32
    return (t + ((v - t) >> sh1)) >> sh2


@pytest.mark.parametrize("seed", [0, 1])
def test_peer_divider_is_exact(seed):
    """The flat kernel finds payload r = v // vpr with one 32x32 multiply-high.
    Check that the planner's multiplier is exact for divisors across the 32-bit
    range and for dividends at every multiple boundary and the extremes."""
    rng = np.random.default_rng(seed)
    ds = list(range(1, 300)) + [(1 << k) + e for k in range(1, 32) for e in (-1, 0, 1)]
    ds += [int(x) for x in rng.integers(1, 1 << 32, 200)]
    ds = sorted({d for d in ds if 1 <= d < (1 << 32)})
    for d in ds:
        p = rog.rog_plan_ptrs([A], 16 * d, 1 << 40, rog.ROG_PATH_MULTI_WG)
        assert p["kernel"] == "flat"
        m, s1, s2 = p["peer_magic"], p["peer_sh1"], p["peer_sh2"]
        vs = {0, 1, d - 1, d, d + 1, (1 << 32) - 1, (1 << 32) - 2}
        q_max = ((1 << 32) - 1) // d
        for q in {1, 2, 3, q_max - 1, q_max} | {int(x) for x in rng.integers(1, q_max + 1, 8)}:
            vs |= {q * d - 1, q * d, q * d + 1}
        vs |= {int(x) for x in rng.integers(0, 1 << 32, 64)}
        for v in vs:
            if 0 <= v < (1 << 32):
                assert _divide(v, m, s1, s2) == v // d, (d, v)
