"""The oracle against its pins (CPU only).

Every pin lives in ``tests/pins.py`` and rests on the pages or on mathematics,
not on the oracle.  The planted-mistake tests at the bottom show that each
plausible slip in a rank-ordered copy (reversed ranks, a stride off by one, a
dropped or extra byte, interleaving, a shifted source index) fails at least
one pin, so the pins can tell a wrong oracle from a right one.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

from oracle import oracle
from deterministic_collective_movement_amd import workloads as wl
from tests import pins

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def c_gather(srcs, buf, start):
    W = len(srcs)
    S = srcs[0].shape[0]
    oracle.gather_c(srcs, buf[start:start + W * S])


def py_gather(srcs, buf, start):
    S = srcs[0].shape[0]
    out = oracle.gather_py([s.tobytes() for s in srcs], S)
    buf[start:start + len(out)] = np.frombuffer(bytes(out), np.uint8)


def join_reference(payloads, S):
    return b"".join(payloads)


# ---------------------------------------------------------------------------
# The C oracle and the pure-Python oracle against the pins
# ---------------------------------------------------------------------------

def test_c_oracle_closed_form():
    pins.pin_closed_form(c_gather)


def test_c_oracle_segments_and_tags():
    pins.pin_segments_and_tags(c_gather)


def test_c_oracle_special_cases():
    pins.pin_special_cases(c_gather)


def test_c_oracle_brute_force_vs_join():
    # W 1..5 x S 0..48 x in-offset 0..15 x out-offset 0..15
    pins.pin_brute_force(c_gather, join_reference, max_W=5, max_S=48, offsets=range(16))


def test_c_oracle_brute_force_vs_python_loop():
    pins.pin_brute_force(c_gather, oracle.gather_py, max_W=5, max_S=48, offsets=(0, 1, 7, 15))


def test_python_oracle_pins():
    pins.all_pins(py_gather, join_reference)


def test_c_oracle_in_place_segment():
    """An output segment that is its own source (src_r == out + r*S) keeps its bytes."""
    W, S = 4, 37
    rng = np.random.default_rng(3)
    out = np.frombuffer(rng.bytes(W * S), np.uint8).copy()
    others = [np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)]
    srcs = [others[0], out[1 * S:2 * S], others[2], out[3 * S:4 * S]]
    want = b"".join([others[0].tobytes(), out[S:2 * S].tobytes(), others[2].tobytes(),
                     out[3 * S:].tobytes()])
    oracle.gather_c(srcs, out)
    assert out.tobytes() == want


def test_c_oracle_aliased_sources():
    """The same payload may feed several ranks."""
    p = np.arange(50, dtype=np.uint8)
    out = np.zeros(150, np.uint8)
    oracle.gather_c([p, p, p], out)
    assert out.tobytes() == p.tobytes() * 3


def test_c_oracle_large_matches_concatenate():
    """A multi-MiB case (ranks x sizes of the bandwidth sweep, scaled down) vs numpy."""
    case = wl.GatherCase(2, 99, 8, 1 * wl.MiB + 5, (0,) * 8, 0)
    payloads = [case.payload(r) for r in range(case.W)]
    out = np.empty(case.W * case.S, np.uint8)
    oracle.gather_c(payloads, out)
    assert np.array_equal(out, np.concatenate(payloads))


# ---------------------------------------------------------------------------
# Batched form
# ---------------------------------------------------------------------------

def test_c_oracle_gather_many_each_tensor_is_its_own_concatenation():
    rng = np.random.default_rng(5)
    W = 4
    sizes = [0, 1, 16, 255, 4096, 3]
    batch = [[np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)] for S in sizes]
    bufs = [pins._guarded(W * S, 1) for S in sizes]
    outs = [b[wl.GUARD + 1: wl.GUARD + 1 + W * S] for b, S in zip(bufs, sizes)]
    oracle.gather_many_c(batch, outs)
    for srcs, out, b, S in zip(batch, outs, bufs, sizes):
        assert out.tobytes() == b"".join(s.tobytes() for s in srcs)
        assert np.all(b[:wl.GUARD + 1] == wl.GUARD_BYTE)
        assert np.all(b[wl.GUARD + 1 + W * S:] == wl.GUARD_BYTE)


def test_c_oracle_gather_many_empty_batch():
    assert oracle.gather_many_c([], []) == []


def test_c_oracle_gather_many_rejects_mixed_W():
    a = np.zeros(4, np.uint8)
    with pytest.raises(ValueError):
        oracle.gather_many_c([[a, a], [a]], [np.zeros(8, np.uint8), np.zeros(4, np.uint8)])


# ---------------------------------------------------------------------------
# Golden fixtures (written by tests/golden/make_golden.py from oracle/ only)
# ---------------------------------------------------------------------------

def _read_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, hexbytes = line.split(None, 1)
            rows[key] = bytes.fromhex(hexbytes)
    return rows


def test_golden_tagged_outputs():
    rows = _read_golden("tagged_gather.txt")
    assert rows, "golden file is empty"
    for key, want in rows.items():
        W, S = (int(x[1:]) for x in key.split("_"))
        payloads = [wl.tagged_payload(r, S) for r in range(W)]
        out = np.empty(W * S, np.uint8)
        oracle.gather_c(payloads, out)
        assert out.tobytes() == want, key
        assert bytes(oracle.gather_py([p.tobytes() for p in payloads], S)) == want, key


def test_golden_page_sizes_are_listed():
    """The pages' own size-test sizes are recorded with their citation."""
    sizes = []
    with open(os.path.join(GOLDEN, "page_sizes.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                sizes.append(int(line))
    assert sizes == [4095, 32 * 1024 + 3, 96 * 1024, 1024 * 1024, 1024 * 1024 + 5]


# ---------------------------------------------------------------------------
# Planted mistakes: each must fail at least one pin
# ---------------------------------------------------------------------------

def _mut_reversed(srcs, buf, start):
    c_gather(srcs[::-1], buf, start)


def _mut_stride_plus_one(srcs, buf, start):
    S = srcs[0].shape[0]
    for r, s in enumerate(srcs):
        lo = start + r * (S + 1)
        n = max(0, min(S, start + len(srcs) * S - lo))
        buf[lo:lo + n] = s[:n]


def _mut_drop_last_byte(srcs, buf, start):
    S = srcs[0].shape[0]
    for r, s in enumerate(srcs):
        buf[start + r * S: start + r * S + max(0, S - 1)] = s[:max(0, S - 1)]


def _mut_extra_byte(srcs, buf, start):
    c_gather(srcs, buf, start)
    S = srcs[0].shape[0]
    if S:
        buf[start + len(srcs) * S] = srcs[-1][-1]


def _mut_interleave(srcs, buf, start):
    W, S = len(srcs), srcs[0].shape[0]
    for r, s in enumerate(srcs):
        buf[start + r: start + W * S: W] = s


def _mut_source_shift(srcs, buf, start):
    S = srcs[0].shape[0]
    for r, s in enumerate(srcs):
        base = s.base if s.base is not None else s
        off = s.__array_interface__["data"][0] - base.__array_interface__["data"][0]
        buf[start + r * S: start + (r + 1) * S] = base[off + 1: off + 1 + S]


def _mut_first_peer_everywhere(srcs, buf, start):
    c_gather([srcs[0]] * len(srcs), buf, start)


MUTANTS = [_mut_reversed, _mut_stride_plus_one, _mut_drop_last_byte, _mut_extra_byte,
           _mut_interleave, _mut_source_shift, _mut_first_peer_everywhere]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_planted_mistake_fails_a_pin(mutant):
    with pytest.raises(AssertionError):
        pins.all_pins(mutant, join_reference)
