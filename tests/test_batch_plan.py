"""The batch planners' chunk layout, checked on the CPU through a shim
compiled from the planner's own source (csrc/rog_plan.cpp): every non-empty
tensor planned once, FLAT tensors first (their chunks go to the XCDs
round-robin, the PEER tensors' after them in XCD runs), first chunks laid end
to end, chunk counts as the kernels expect, and the sum batch's tensors in
the caller's order."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from deterministic_collective_movement_amd import build as b
from deterministic_collective_movement_amd import rog

HERE = os.path.dirname(os.path.abspath(__file__))
MAXB = 32


def sum_forms(W, source_bytes):
    """The header's rule for a sum: streamed loads from 128 MiB of sources,
    and then shared granules.  (nt, granule form)"""
    nt = source_bytes >= 128 << 20
    return nt, nt


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    hipcc = shutil.which("hipcc") or os.path.join(b.ROCM, "bin", "hipcc")
    so = str(tmp_path_factory.mktemp("plan") / "libplanshim.so")
    subprocess.check_call([hipcc, "-x", "hip", "-O2", "-std=c++17", "-fPIC", "-shared",
                           "--offload-arch=gfx950", "-Wno-unused-command-line-argument",
                           "-I", b.INCLUDE, "-I", b.CSRC, os.path.join(HERE, "plan_shim.cpp"),
                           os.path.join(b.CSRC, "rog_plan.cpp"), "-o", so],
                          stderr=subprocess.DEVNULL)
    return ctypes.CDLL(so)


U64 = ctypes.c_uint64 * 64
U32 = ctypes.c_uint32 * 64


def plan_batch(shim, tensors, W):
    """tensors: [(src addresses, out address, S)] -> (status, planned list, meta)."""
    keep = [(ctypes.c_void_p * W)(*srcs) for srcs, _, _ in tensors]
    descs = (rog.rog_gather_desc * max(1, len(tensors)))()
    for i, (srcs, o, S) in enumerate(tensors):
        descs[i].srcs = ctypes.cast(keep[i], ctypes.POINTER(ctypes.c_void_p))
        descs[i].out = ctypes.c_void_p(o)
        descs[i].bytes_per_rank = S
    n_out = ctypes.c_uint32()
    out, S, flat, nch, first = U64(), U64(), U32(), U32(), U32()
    srcs = (ctypes.c_uint64 * (MAXB * 8))()
    meta = (ctypes.c_uint32 * 4)()
    status = shim.rog_test_plan_batch(descs, len(tensors), W, ctypes.byref(n_out), out, S, flat, nch, first,
                                      srcs, meta)
    planned = [dict(out=out[k], S=S[k], flat=flat[k], n_chunks=nch[k], first=first[k],
                    srcs=tuple(srcs[k * W + r] for r in range(W))) for k in range(n_out.value)]
    return status, planned, list(meta)


def _chunks(srcs, o, S, W):
    """(FLAT?, chunks, line-aligned FLAT?).  A FLAT tensor's first chunk is
    short by (o % 128) / 16 vectors so the others start on o's 128-byte lines."""
    flat = ((o | S | _or(srcs)) & 15) == 0
    if flat:
        n_vec = W * S // 16
        shift = (o % 128) // 16
        return True, -(-(n_vec + shift) // 64), ((o | S | _or(srcs)) & 127) == 0
    return False, max(1, -(-(S // 16) // 64)) * W, False


def _or(xs):
    v = 0
    for x in xs:
        v |= x
    return v


BASE = 1 << 40


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(data=st.data(), n=st.integers(0, 12), W=st.sampled_from([1, 2, 4, 8]))
def test_gather_batch_layout(shim, data, n, W):
    tensors = []
    for t in range(n):
        S = data.draw(st.one_of(st.just(0), st.integers(1, 5000),
                                st.sampled_from([16, 1024, 4096, 65536, 1 << 20, 24 << 20])))
        off = data.draw(st.sampled_from([0, 0, 16, 1, 3, 8, 48, 128]))
        base = BASE + t * (1 << 32)
        srcs = [base + r * (1 << 28) + off for r in range(W)]
        o = base + (W + 1) * (1 << 28) + data.draw(st.sampled_from([0, 16, 1, 5, 80, 128]))
        tensors.append((srcs, o, S))
    status, planned, meta = plan_batch(shim, tensors, W)
    assert status == 0
    want = [(tuple(s), o, S) + _chunks(s, o, S, W) for s, o, S in tensors if S]
    # line-aligned FLAT tensors first (round-robin), then the rest (XCD runs),
    # each group in the caller's order
    order = [x[:5] for x in want if x[5]] + [x[:5] for x in want if not x[5]]
    assert [(p["srcs"], p["out"], p["S"], bool(p["flat"]), p["n_chunks"]) for p in planned] == order
    nxt = 0
    for p in planned:
        assert p["first"] == nxt
        nxt += p["n_chunks"]
    assert meta[0] == nxt
    assert meta[1] == sum(x[4] for x in want if x[5])
    assert meta[2] == nxt            # one wave per chunk while the grid is not capped
    assert meta[3] == int(W * sum(S for _, _, S in tensors) >= 128 << 20)   # streamed loads from 128 MiB


def test_gather_batch_all_empty(shim):
    status, planned, meta = plan_batch(shim, [([BASE], BASE + (1 << 30), 0)] * 3, 1)
    assert status == 0 and planned == [] and meta[0] == 0 and meta[2] == 0


def plan_reduce_batch(shim, tensors, W, dtype):
    keep = [(ctypes.c_void_p * W)(*srcs) for srcs, _, _ in tensors]
    descs = (rog.rog_reduce_desc * max(1, len(tensors)))()
    for i, (srcs, o, cnt) in enumerate(tensors):
        descs[i].srcs = ctypes.cast(keep[i], ctypes.POINTER(ctypes.c_void_p))
        descs[i].out = ctypes.c_void_p(o)
        descs[i].count = cnt
    n_out = ctypes.c_uint32()
    out, count, nch, first = U64(), U64(), U32(), U32()
    meta = (ctypes.c_uint32 * 4)()
    status = shim.rog_test_plan_reduce_batch(descs, len(tensors), W, dtype, ctypes.byref(n_out), out, count, nch,
                                             first, meta)
    planned = [dict(out=out[k], count=count[k], n_chunks=nch[k], first=first[k]) for k in range(n_out.value)]
    return status, planned, list(meta)


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(data=st.data(), n=st.integers(0, 12), W=st.sampled_from([1, 3, 4]), dtype=st.sampled_from([0, 1, 2]))
def test_reduce_batch_layout(shim, data, n, W, dtype):
    es = 4 if dtype == 0 else 2
    tensors = []
    for t in range(n):
        cnt = data.draw(st.one_of(st.just(0), st.integers(1, 100_000), st.just(24 << 20)))
        base = BASE + t * (1 << 33)
        srcs = [base + r * (1 << 29) + es * data.draw(st.integers(0, 7)) for r in range(W)]
        o = base + (W + 1) * (1 << 29) + es * data.draw(st.integers(0, 7))
        tensors.append((srcs, o, cnt))
    status, planned, meta = plan_reduce_batch(shim, tensors, W, dtype)
    assert status == 0
    want = [(o, cnt, max(1, -(-(cnt * es // 16) // 64))) for _, o, cnt in tensors if cnt]
    assert [(p["out"], p["count"], p["n_chunks"]) for p in planned] == want   # the caller's order
    nxt = 0
    for p in planned:
        assert p["first"] == nxt
        nxt += p["n_chunks"]
    assert meta[0] == nxt and meta[1] == nxt
    source_bytes = sum(W * cnt * es for _, _, cnt in tensors)
    nt, granule = sum_forms(W, source_bytes)
    assert meta[2] == int(nt) and meta[3] == int(granule)


def _lookup(shim, tensors, W, chunks):
    keep = [(ctypes.c_void_p * W)(*srcs) for srcs, _, _ in tensors]
    descs = (rog.rog_gather_desc * max(1, len(tensors)))()
    for i, (srcs, o, S) in enumerate(tensors):
        descs[i].srcs = ctypes.cast(keep[i], ctypes.POINTER(ctypes.c_void_p))
        descs[i].out = ctypes.c_void_p(o)
        descs[i].bytes_per_rank = S
    q = (ctypes.c_uint32 * len(chunks))(*chunks)
    got = (ctypes.c_uint32 * len(chunks))()
    shift = ctypes.c_uint32()
    assert shim.rog_test_batch_lookup(descs, len(tensors), W, q, len(chunks), got, ctypes.byref(shift)) == 0
    return list(got), shift.value


def _owner(first, c):
    import bisect
    return bisect.bisect_right(first, c) - 1


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(data=st.data(), n=st.integers(1, 32), W=st.sampled_from([1, 2, 4]))
def test_batch_lookup_finds_every_chunks_tensor(shim, data, n, W):
    """The kernels' chunk -> tensor lookup (a bucket table, then a search over
    the tensors that meet the bucket) against a plain search over the first
    chunks: every chunk of small batches, and the first, last and random
    chunks of every tensor of large ones (up to 2^28 chunks)."""
    tensors = []
    for t in range(n):
        S = data.draw(st.one_of(st.just(0), st.integers(1, 3000),
                                st.sampled_from([16, 1024, 65536, 1 << 20, 1 << 24, 1 << 28])))
        base = BASE + t * (1 << 34)
        srcs = [base + r * (1 << 30) for r in range(W)]
        tensors.append((srcs, base + (W + 1) * (1 << 30) + data.draw(st.sampled_from([0, 16, 3])), S))
    status, planned, meta = plan_batch(shim, tensors, W)
    assert status == 0
    if not planned:
        return
    first = [p["first"] for p in planned]
    total = meta[0]
    if total <= 20000:
        chunks = list(range(total))
    else:
        chunks = []
        for p in planned:
            lo, hi = p["first"], p["first"] + p["n_chunks"]
            chunks += [lo, hi - 1, (lo + hi) // 2]
            chunks += [data.draw(st.integers(lo, hi - 1)) for _ in range(3)]
    got, shift = _lookup(shim, tensors, W, chunks)
    assert ((total - 1) >> shift) < 256
    assert got == [_owner(first, c) for c in chunks]


def test_batch_lookup_many_small_tensors_in_one_bucket(shim):
    """Thirty-one one-chunk tensors and one huge one: the small ones share the
    first bucket, and the search among them still finds each."""
    W = 1
    tensors = [([BASE + t * (1 << 32)], BASE + t * (1 << 32) + (1 << 31), 1024) for t in range(31)]
    tensors.append(([BASE + 40 * (1 << 32)], BASE + 41 * (1 << 32), 1 << 30))
    status, planned, meta = plan_batch(shim, tensors, W)
    assert status == 0 and len(planned) == 32
    first = [p["first"] for p in planned]
    chunks = list(range(0, 64)) + [meta[0] - 1, meta[0] // 2]
    got, shift = _lookup(shim, tensors, W, chunks)
    assert shift > 0
    assert got == [_owner(first, c) for c in chunks]


@settings(max_examples=80, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(data=st.data(), n=st.integers(1, 32), W=st.sampled_from([1, 3]))
def test_reduce_batch_lookup_finds_every_chunks_tensor(shim, data, n, W):
    tensors = []
    for t in range(n):
        cnt = data.draw(st.one_of(st.just(0), st.integers(1, 20_000), st.sampled_from([1 << 16, 1 << 22, 1 << 27])))
        base = BASE + t * (1 << 34)
        tensors.append(([base + r * (1 << 30) for r in range(W)], base + (W + 1) * (1 << 30), cnt))
    status, planned, _ = plan_reduce_batch(shim, tensors, W, 0)
    assert status == 0
    if not planned:
        return
    first = [p["first"] for p in planned]
    chunks = []
    for p in planned:
        lo, hi = p["first"], p["first"] + p["n_chunks"]
        chunks += [lo, hi - 1, (lo + hi) // 2, data.draw(st.integers(lo, hi - 1))]
    keep = [(ctypes.c_void_p * W)(*srcs) for srcs, _, _ in tensors]
    descs = (rog.rog_reduce_desc * len(tensors))()
    for i, (srcs, o, cnt) in enumerate(tensors):
        descs[i].srcs = ctypes.cast(keep[i], ctypes.POINTER(ctypes.c_void_p))
        descs[i].out = ctypes.c_void_p(o)
        descs[i].count = cnt
    q = (ctypes.c_uint32 * len(chunks))(*chunks)
    got = (ctypes.c_uint32 * len(chunks))()
    assert shim.rog_test_reduce_batch_lookup(descs, len(tensors), W, 0, q, len(chunks), got) == 0
    assert list(got) == [_owner(first, c) for c in chunks]


def test_sum_granule_group_by_W(shim):
    """The granule form keeps 2 sources' granules in flight for W <= 2, 4 for
    W = 3 and 8 from W = 4 on (the measured rule)."""
    shim.rog_test_sum_granule_group.restype = ctypes.c_uint32
    shim.rog_test_sum_granule_group.argtypes = [ctypes.c_uint32]
    got = [shim.rog_test_sum_granule_group(W) for W in range(1, 65)]
    assert got == [2, 2, 4] + [8] * 61
