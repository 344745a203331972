"""Property tests of the host planner (rog_plan / rog_reduce_plan, no HIP
calls): random pointer layouts, sizes, W and paths drawn by hypothesis, and
the status and launch shape each returns compared with the rules that
include/rog.h states, written out here independently of csrc/."""
from __future__ import annotations

import ctypes

from hypothesis import HealthCheck, given, settings, strategies as st

from deterministic_collective_movement_amd import rog

U64 = (1 << 64) - 1
OK, INVALID, OVERLAP, TOO_LARGE = (rog.ROG_OK, rog.ROG_ERR_INVALID_ARGUMENT,
                                   rog.ROG_ERR_OVERLAP, rog.ROG_ERR_TOO_LARGE)
MAXW = rog.rog_max_peers()
SINGLE_MAX = rog.rog_single_wg_max_bytes()
RSINGLE_MAX = rog.rog_reduce_single_wg_max_bytes()


def sum_forms(W, source_bytes):
    """The header's rule for a sum: streamed loads from 128 MiB of sources,
    and then shared granules.  (nt, granule form)"""
    nt = source_bytes >= 128 << 20
    return nt, nt


def overlap(a, na, b, nb):
    return na > 0 and nb > 0 and a < b + nb and b < a + na


def gather_rules(srcs, W, S, out, path):
    """Status of a gather per include/rog.h, checks in the header's order."""
    if path not in (0, 1, 2) or W < 1 or W > MAXW:
        return INVALID
    if S == 0:
        return OK
    if out == 0 or any(s == 0 for s in srcs):
        return INVALID
    if S > U64 // W:
        return TOO_LARGE
    total = W * S
    if total >= 1 << 36:
        return TOO_LARGE
    if out > U64 - total:
        return INVALID
    for r, s in enumerate(srcs):
        if s > U64 - S:
            return INVALID
        if overlap(s, S, out, total) and s != out + r * S:
            return OVERLAP
    return OK


def reduce_rules(srcs, W, n, es, out, path):
    if path not in (0, 1, 2) or W < 1 or W > MAXW:
        return INVALID
    if n == 0:
        return OK
    if out == 0 or any(s == 0 for s in srcs):
        return INVALID
    if n > U64 // es:
        return TOO_LARGE
    nb = n * es
    if nb >= 1 << 36:
        return TOO_LARGE
    if out % es or out > U64 - nb:
        return INVALID
    for s in srcs:
        if s % es or s > U64 - nb:
            return INVALID
        if overlap(s, nb, out, nb) and s != out:
            return OVERLAP
    return OK


def plan(srcs, W, S, out, path):
    info = rog.rog_plan_info()
    status = rog.lib().rog_plan(rog._ptr_array(srcs), W, S, ctypes.c_void_p(out), path, ctypes.byref(info))
    return status, info


def rplan(srcs, W, n, dt, out, path):
    info = rog.rog_plan_info()
    status = rog.lib().rog_reduce_plan(rog._ptr_array(srcs), W, n, dt, ctypes.c_void_p(out), path,
                                       ctypes.byref(info))
    return status, info


# Pointer layouts: a base region, each pointer near it at a small random offset
# (so overlaps, exact in-place segments and alignment classes all occur), plus
# occasional NULLs and addresses near the top of the address space.
BASE = 1 << 40
sizes = st.one_of(st.integers(0, 64), st.integers(0, 1 << 22), st.sampled_from([16, 256, 4096, (1 << 20) + 3,
                                                                                   1 << 35, (1 << 36) - 16, U64 // 2]))
addr_near = st.one_of(st.integers(BASE - (1 << 23), BASE + (1 << 23)), st.just(0),
                      st.integers(U64 - (1 << 12), U64))


@settings(max_examples=700, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(W=st.integers(0, MAXW + 1), S=sizes, path=st.sampled_from([0, 1, 2, 3]), data=st.data())
def test_gather_plan_matches_the_rules(W, S, path, data):
    out = data.draw(addr_near, label="out")
    in_place = data.draw(st.lists(st.booleans(), min_size=max(W, 1), max_size=max(W, 1)), label="in_place")
    srcs = []
    for r in range(max(W, 1)):
        if in_place[r] and out:
            srcs.append((out + r * S) & U64)
        else:
            srcs.append(data.draw(addr_near, label="src%d" % r))
    srcs = srcs[:W] if W else [BASE]
    status, info = plan(srcs, W, S, out, path)
    want = gather_rules(srcs, W, S, out, path)
    assert status == want, (status, want, W, S, out, srcs, path)
    if status != OK:
        return
    total = W * S
    resolved = path if path else (1 if total <= SINGLE_MAX else 2)
    assert info.path == resolved
    if S == 0:
        assert info.kernel == rog.ROG_KERNEL_NONE and info.grid == 0
        return
    flat = ((out | S | _or(srcs)) & 15) == 0
    assert info.kernel == (rog.ROG_KERNEL_FLAT if flat else rog.ROG_KERNEL_PEER)
    assert info.grid >= 1 and info.grid * info.block < (1 << 32)
    if info.path == 1:
        assert info.grid == 1 and 64 <= info.block <= 1024 and info.block % 64 == 0
    if flat and info.path == 2:
        # one-wave workgroups over 1 KiB chunks, the first short by the
        # output's vectors past a 128-byte line (none from 2^31 vectors on)
        n_vec = total // 16
        k = (out % 128) // 16 if n_vec < (1 << 31) else 0
        assert info.block == 64
        assert info.grid == min(max(1, -(-(n_vec + k) // 64)), 0xFFFFFFFF // 64), (n_vec, k, info.grid)
    if not flat:
        mask = sum(1 << r for r, s in enumerate(srcs) if ((s | (out + r * S)) & 15) == 0)
        assert info.vec_ok_mask == mask
    assert bool(info.flags & rog.ROG_PLAN_NT_LOADS) == (total >= 128 << 20)
    shifted = (not flat and info.path == 2 and total >= 128 << 20
               and any(shared_granules(s, out + r * S, S, PEER_MODE) for r, s in enumerate(srcs)))
    assert bool(info.flags & rog.ROG_PLAN_SHIFTED_LOADS) == shifted


# The multi-WG PEER body starts at the first 256-byte boundary of its output;
# where the loads stream past the caches, a source sitting m bytes past a
# 16-byte granule there is read as aligned granules shared between lanes when
# m is odd or 2 mod 4 (mode 1, as built); mode 2 would take every m != 0.
# (The sum takes its granule form exactly when its loads stream.)
PEER_MODE, REDUCE_MODE = 1, 2


def shared_granules(src, dst, nbytes, mode):
    head = (256 - dst % 256) % 256
    if nbytes < head + 16:
        return False              # no body
    m = (src + head) % 16
    return m != 0 if mode == 2 else m % 4 != 0


def _or(xs):
    v = 0
    for x in xs:
        v |= x
    return v


@settings(max_examples=700, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(W=st.integers(0, MAXW + 1), n=sizes, dt=st.sampled_from([0, 1, 2]), path=st.sampled_from([0, 1, 2, 3]),
       data=st.data())
def test_reduce_plan_matches_the_rules(W, n, dt, path, data):
    es = 4 if dt == 0 else 2
    out = data.draw(addr_near, label="out")
    srcs = [out if (out and data.draw(st.booleans(), label="in_place%d" % r)) else data.draw(addr_near, label="src%d" % r)
            for r in range(max(W, 1))]
    srcs = srcs[:W] if W else [BASE]
    status, info = rplan(srcs, W, n, dt, out, path)
    want = reduce_rules(srcs, W, n, es, out, path)
    assert status == want, (status, want, W, n, es, out, srcs, path)
    if status != OK or n == 0:
        return
    nb = n * es
    assert info.kernel == rog.ROG_KERNEL_REDUCE and info.units == n
    resolved = path if path else (1 if W * nb <= RSINGLE_MAX else 2)
    assert info.path == resolved
    if resolved == 2:
        assert info.block == 64 and info.grid == min(max(1, -(-(nb // 16) // 64)), 0xFFFFFFFF // 64)
    else:
        assert info.grid == 1 and info.block == min(1024, max(64, -(-(-(-nb // 16)) // 64) * 64))
    nt, granule = sum_forms(W, W * nb)
    assert bool(info.flags & rog.ROG_PLAN_NT_LOADS) == nt
    assert bool(info.flags & rog.ROG_PLAN_SHIFTED_LOADS) == (resolved == 2 and granule)


def test_shared_granule_examples():
    """Hand-worked cases of the rule above."""
    g = BASE                                 # 256-byte aligned
    for mode in (PEER_MODE, REDUCE_MODE):
        assert not shared_granules(g, g, 1 << 20, mode)          # m = 0
        assert shared_granules(g + 2, g, 1 << 20, mode)          # bf16 one element off: m = 2
        assert shared_granules(g + 1, g + 3, 1 << 20, mode)      # head 253: m = (1 + 253) % 16 = 14
        assert not shared_granules(g + 1, g + 3, 253 + 15, mode)  # body empty
        assert shared_granules(g, g + 255, 1 << 20, mode)        # head 1: m = 1
    assert not shared_granules(g + 4, g, 1 << 20, PEER_MODE)     # m = 4: the gather keeps the unaligned load
    assert shared_granules(g + 4, g, 1 << 20, REDUCE_MODE)


def test_bad_dtype_is_invalid():
    assert rplan([BASE], 1, 16, 3, BASE + 4096, 0)[0] == INVALID
