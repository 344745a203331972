"""Pins for the rank-ordered gather: checks fixed by the pages and by mathematics,
independent of any implementation under test.

A ``gather`` under test has the signature ``gather(srcs, buf, out_off)``: it
copies the W equal-length uint8 payloads ``srcs`` into ``buf[out_off:out_off+W*S]``
and must leave every other byte of ``buf`` alone.

What each pin rests on (RL-Align/RL-Kernel PR #491, "perf(cuda): vectorize the
deterministic all-gather copy and right-size its single-block path"):

* closed form -- the copy puts the same bytes where an all-gather does, i.e.
  the output is the concatenation of the payloads in rank order ("What",
  copy_rank_ordered bullet; "Tests": compared with NCCL's all-gather);
* per-segment invariant and peer tags -- segment r of the output is payload r;
* guards -- bytes before and after the output are untouched (review threads on
  the size test: 0xA5 prefix sentinel and a trailing guard);
* sources unchanged -- a gather only reads its payloads.
"""
from __future__ import annotations

import itertools

import numpy as np

from deterministic_collective_movement_amd import workloads as wl


def _guarded(total: int, off: int) -> np.ndarray:
    return np.full(wl.GUARD + off + total + wl.GUARD, wl.GUARD_BYTE, dtype=np.uint8)


def _payloads_in_buffers(payloads, offs):
    bufs, views = [], []
    for p, o in zip(payloads, offs):
        b = _guarded(p.shape[0], o)
        b[wl.GUARD + o: wl.GUARD + o + p.shape[0]] = p
        bufs.append(b)
        views.append(b[wl.GUARD + o: wl.GUARD + o + p.shape[0]])
    return bufs, views


def run_case(gather, payloads, in_offs, out_off):
    """Run ``gather`` on payloads placed at the given offsets; return (buf, out view, srcs)."""
    W = len(payloads)
    S = payloads[0].shape[0]
    src_bufs, srcs = _payloads_in_buffers(payloads, in_offs)
    before = [b.copy() for b in src_bufs]
    buf = _guarded(W * S, out_off)
    start = wl.GUARD + out_off
    gather(srcs, buf, start)
    for b, a in zip(src_bufs, before):
        assert np.array_equal(b, a), "a source buffer changed"
    assert np.all(buf[:start] == wl.GUARD_BYTE), "prefix guard overwritten"
    assert np.all(buf[start + W * S:] == wl.GUARD_BYTE), "suffix guard overwritten"
    return buf, buf[start:start + W * S]


def pin_closed_form(gather, seed=7):
    """Output == b"".join(payloads) == numpy.concatenate(payloads)."""
    rng = np.random.default_rng(seed)
    for W, S in [(1, 1), (2, 3), (3, 16), (4, 31), (5, 100), (8, 257), (2, 4096 + 5)]:
        payloads = [np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)]
        _, out = run_case(gather, payloads, [0] * W, 0)
        assert out.tobytes() == b"".join(p.tobytes() for p in payloads), (W, S)
        assert np.array_equal(out, np.concatenate(payloads)), (W, S)


def pin_segments_and_tags(gather):
    """Segment r equals payload r, and every byte decodes to its (rank, index) tag."""
    for W, S in [(2, 1), (3, 5), (4, 17), (8, 300), (5, 251), (7, 1000)]:
        payloads = [wl.tagged_payload(r, S) for r in range(W)]
        _, out = run_case(gather, payloads, [r % 4 for r in range(W)], 3)
        for r in range(W):
            seg = out[r * S:(r + 1) * S]
            i = np.arange(S, dtype=np.int64)
            assert np.array_equal(seg, ((r * 131 + i * 7 + 1) % 251).astype(np.uint8)), (W, S, r)


def pin_special_cases(gather):
    """S = 0 writes nothing; W = 1 is a plain copy."""
    payloads = [np.zeros(0, np.uint8) for _ in range(3)]
    buf, out = run_case(gather, payloads, [0, 1, 2], 5)
    assert out.shape[0] == 0
    p = np.arange(1, 40, dtype=np.uint8)
    _, out = run_case(gather, [p], [3], 1)
    assert np.array_equal(out, p)


def pin_brute_force(gather, reference, max_W=5, max_S=48, offsets=range(16), seed=11):
    """Every W <= max_W, S <= max_S and in/out offset pair against ``reference``
    (an independent implementation: the pure-Python loop or bytes.join)."""
    rng = np.random.default_rng(seed)
    for W in range(1, max_W + 1):
        for S in range(0, max_S + 1):
            payloads = [np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)]
            want = reference([p.tobytes() for p in payloads], S)
            for io, oo in itertools.product(offsets, offsets):
                _, out = run_case(gather, payloads, [io] * W, oo)
                assert out.tobytes() == bytes(want), (W, S, io, oo)


def all_pins(gather, reference, brute=dict(max_W=3, max_S=20, offsets=(0, 1, 15))):
    pin_closed_form(gather)
    pin_segments_and_tags(gather)
    pin_special_cases(gather)
    pin_brute_force(gather, reference, **brute)
