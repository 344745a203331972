"""The rank-ordered sum's C ABI on the CPU: argument validation, in-place and
overlap rules, path dispatch and grid sizing (include/rog.h, rog_reduce*).
rog_reduce_plan never calls HIP, and every rog_reduce call below fails
validation or has nothing to do, so none of them launches a kernel."""
from __future__ import annotations

import ctypes

import pytest

from deterministic_collective_movement_amd import rog

A = 1 << 33
F32, BF16, F16 = rog.ROG_DTYPE_F32, rog.ROG_DTYPE_BF16, rog.ROG_DTYPE_F16
OK, INVALID, OVERLAP, TOO_LARGE = (rog.ROG_OK, rog.ROG_ERR_INVALID_ARGUMENT,
                                   rog.ROG_ERR_OVERLAP, rog.ROG_ERR_TOO_LARGE)


def st(srcs, count, out, dtype=F32, path=rog.ROG_PATH_AUTO, W=None):
    info = rog.rog_plan_info()
    arr = None if srcs is None else rog._ptr_array(srcs)
    return int(rog.lib().rog_reduce_plan(arr, len(srcs) if W is None else W, count, dtype,
                                         ctypes.c_void_p(out), path, ctypes.byref(info)))


def test_declared_and_exported():
    lib = rog.lib()
    for name in ("rog_reduce", "rog_reduce_ex", "rog_reduce_plan", "rog_reduce_single_wg_max_bytes"):
        assert hasattr(lib, name), name
    assert rog.rog_reduce_single_wg_max_bytes() > 0


def test_invalid_arguments():
    assert st(None, 16, A, W=2) == INVALID
    assert st([A], 16, A + 4096, W=0) == INVALID
    M = rog.rog_max_peers()
    assert st([A + 256 * i for i in range(M + 1)], 16, 2 * A) == INVALID
    assert st([A + 256 * i for i in range(M)], 16, 2 * A) == OK
    assert st([A, 0], 16, 2 * A) == INVALID
    assert st([A, A + 64], 16, 0) == INVALID
    assert st([A], 16, 2 * A, dtype=3) == INVALID            # unknown dtype
    assert st([A], 16, 2 * A, dtype=-1) == INVALID
    assert st([A], 16, 2 * A, path=5) == INVALID
    assert rog.lib().rog_reduce_plan(rog._ptr_array([A]), 1, 16, F32, ctypes.c_void_p(2 * A), 0, None) == INVALID


def test_element_alignment():
    # binary32 elements need 4-byte addresses, bf16 2-byte ones; nothing more
    assert st([A + 2], 16, 2 * A, F32) == INVALID
    assert st([A], 16, 2 * A + 2, F32) == INVALID
    assert st([A + 4, A + 4096 + 12], 16, 2 * A + 8, F32) == OK
    assert st([A + 1], 16, 2 * A, BF16) == INVALID
    assert st([A], 16, 2 * A + 3, BF16) == INVALID
    assert st([A + 2, A + 4096 + 6], 16, 2 * A + 14, BF16) == OK
    assert st([A + 1], 16, 2 * A, F16) == INVALID
    assert st([A + 2, A + 4096 + 6], 16, 2 * A + 14, F16) == OK


def test_zero_count_is_a_no_op_even_with_null_pointers():
    assert st([0, 0], 0, 0) == OK
    p = rog.rog_reduce_plan_ptrs([0, 0, 0], 0, F32, 0)
    assert p["kernel"] == "none" and p["grid"] == 0
    rog.rog_reduce_ptrs([0, 0], 0, BF16, 0)                  # nothing enqueued, no HIP call


def test_too_large():
    big = (1 << 64) - 1
    assert st([A], big // 2 + 1, 1 << 40, F32) == TOO_LARGE  # count * 4 overflows
    assert st([A], 1 << 34, 1 << 40, F32) == TOO_LARGE       # 2^36 bytes
    assert st([A], (1 << 34) - 4, 1 << 40, F32) == OK
    assert st([A], 1 << 35, 1 << 40, BF16) == TOO_LARGE


def test_address_wrap_is_invalid():
    top = (1 << 64) - 64
    assert st([top], 128, A) == INVALID
    assert st([A], 128, top) == INVALID


def test_in_place_and_overlap_rules():
    n = 1000                                                  # 4000 bytes of binary32
    out = 1 << 24
    assert st([out, A], n, out) == OK                         # out is srcs[0]
    assert st([A, out, out], n, out) == OK                    # out is two of the sources
    assert st([A, out + 4], n, out) == OVERLAP                # shifted by one element
    assert st([out - 4000, A], n, out) == OK                  # touching, not overlapping
    assert st([out - 3996, A], n, out) == OVERLAP
    assert st([A, A, A], n, out) == OK                        # aliased sources


def test_auto_path_follows_the_bound_on_source_bytes_inclusively():
    bound = rog.rog_reduce_single_wg_max_bytes()
    for W in (1, 2, 8):
        srcs = [A + r * (1 << 28) for r in range(W)]
        for dtype, es in ((F32, 4), (BF16, 2)):
            n = bound // (W * es)              # W * n * es == bound exactly
            assert rog.rog_reduce_plan_ptrs(srcs, n, dtype, 1 << 40)["path"] == "single_wg", (W, es)
            assert rog.rog_reduce_plan_ptrs(srcs, n + 1, dtype, 1 << 40)["path"] == "multi_wg", (W, es)


@pytest.mark.parametrize("count,dtype", [(1, F32), (4096, F32), (100001, BF16), (1 << 24, BF16), (7, BF16)])
def test_grid_sizes(count, dtype):
    es = 4 if dtype == F32 else 2
    srcs = [A + 2, A + (1 << 30) + 6] if dtype == BF16 else [A, A + (1 << 30)]
    p = rog.rog_reduce_plan_ptrs(srcs, count, dtype, 1 << 34, rog.ROG_PATH_MULTI_WG)
    assert p["kernel"] == "reduce" and p["block"] == 64 and p["units"] == count
    # one wave per 1 KiB chunk of the at most count * es / 16 body vectors
    assert p["grid"] == max(1, -(-(count * es // 16) // 64))
    s = rog.rog_reduce_plan_ptrs(srcs, count, dtype, 1 << 34, rog.ROG_PATH_SINGLE_WG)
    assert s["grid"] == 1 and s["block"] == min(1024, max(64, -(-(-(-count * es // 16)) // 64) * 64))


def test_nt_loads_and_granule_form_follow_source_bytes():
    # loads stream past the caches from 128 MiB of sources, whatever W, and
    # the granule form comes with them
    for W in (1, 2, 3, 4, 8, 64):
        n = -(-(128 << 20) // (2 * W))
        srcs = [A + i * (1 << 30) for i in range(W)]
        p = rog.rog_reduce_plan_ptrs(srcs, n, BF16, 1 << 45)
        assert p["nt_loads"] and p["shifted_loads"], W
        p = rog.rog_reduce_plan_ptrs(srcs, n - 64, BF16, 1 << 45)
        assert not p["nt_loads"] and not p["shifted_loads"], W


def test_binding_errors_map_to_exceptions():
    with pytest.raises(rog.RogArgumentError):
        rog.rog_reduce_ptrs([A + 1], 16, F32, 2 * A)
    with pytest.raises(rog.RogArgumentError):
        rog.rog_reduce_ptrs([A, A + 8], 16, F32, A + 8)


# ---------------------------------------------------------------------------
# rog_reduce_many validation (every case returns before any HIP call)
# ---------------------------------------------------------------------------

def many_status(batch, counts, outs, W, dtype=F32, n=None):
    keep = [rog._ptr_array(p) for p in batch]
    descs = (rog.rog_reduce_desc * max(1, len(outs)))()
    for t in range(len(outs)):
        descs[t].srcs = ctypes.cast(keep[t], ctypes.POINTER(ctypes.c_void_p))
        descs[t].out = ctypes.c_void_p(outs[t])
        descs[t].count = counts[t]
    return int(rog.lib().rog_reduce_many(descs, len(outs) if n is None else n, W, dtype, None))


def test_reduce_many_validation():
    assert rog.lib().rog_reduce_many(None, 0, 2, F32, None) == OK           # empty batch
    assert rog.lib().rog_reduce_many(None, 1, 2, F32, None) == INVALID      # NULL descriptors
    assert many_status([[A, A + 4096]], [16], [1 << 36], 2, dtype=7) == INVALID
    assert many_status([[A]], [16], [1 << 36], 0) == INVALID
    n_max, p_max = rog.rog_max_batch(), rog.rog_max_batch_pointers()
    assert many_status([[A]] * (n_max + 1), [0] * (n_max + 1), [0] * (n_max + 1), 1) == TOO_LARGE
    W = p_max // 4 + 1
    assert many_status([[A] * W] * 4, [0] * 4, [0] * 4, W) == TOO_LARGE
    # per-tensor rules: alignment, partial overlap with its own output
    assert many_status([[A + 2]], [16], [1 << 36], 1, F32) == INVALID
    assert many_status([[A, (1 << 36) + 4]], [16], [1 << 36], 2) == OVERLAP
    # across tensors: outputs, and an output over another tensor's source
    o1, o2 = 1 << 36, (1 << 36) + (1 << 20)
    assert many_status([[A], [A + 64]], [16, 16], [o1, o1 + 32], 1) == OVERLAP
    assert many_status([[A], [o1 + 8]], [16, 16], [o1, o2], 1) == OVERLAP
    assert many_status([[A, o2], [A, A]], [16, 16], [o1, o2], 2) == OVERLAP  # o2 is tensor 0's source
    assert many_status([[0, 0], [0, 0]], [0, 0], [0, 0], 2) == OK           # all empty: nothing enqueued
    # (valid non-empty batches launch a kernel: the GPU tests run them)
