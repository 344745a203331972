"""The GPU parity harness itself (tests/gpu_cases.py), checked on the CPU.

Every GPU parity test ends in Placed.check or PlacedReduce.check.  Here those
checks run on CPU tensors standing in for device buffers: a correct result
must pass, and each planted mistake must be caught -- a wrong output byte, a
touched guard byte on either side, a changed source byte, a sum one ulp off,
a finite value where the oracle has a NaN (and the reverse), a byte written
past an in-place sum's output, and one wrong tensor of a batch.  (The pages'
own benchmark tests are checked the same way: each is shown to fail under its
mutation -- RL-Align/RL-Kernel PR #491, the author's replies on the benchmark
tests.)"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from deterministic_collective_movement_amd import workloads as wl
from oracle import oracle
from tests import gpu_cases as gc

CPU = torch.device("cpu")


def _gather(W=3, S=37, in_offs=(1, 0, 3), out_off=5, seed=11):
    rng = np.random.default_rng(seed)
    payloads = [rng.integers(0, 256, S, dtype=np.uint8) for _ in range(W)]
    p = gc.Placed(payloads, list(in_offs), out_off, CPU)
    return p, payloads


def _write_correct(p, payloads):
    """What a correct gather leaves behind: the concatenation, nothing else."""
    p.out.copy_(torch.from_numpy(np.concatenate(payloads)))


def test_correct_gather_passes():
    p, payloads = _gather()
    _write_correct(p, payloads)
    p.check("correct")


def test_untouched_output_fails():
    p, _ = _gather()
    with pytest.raises(AssertionError, match="output byte 0"):
        p.check("nothing written")


@pytest.mark.parametrize("where", ["first", "middle", "last"])
def test_wrong_output_byte_fails(where):
    p, payloads = _gather()
    _write_correct(p, payloads)
    i = {"first": 0, "middle": p.W * p.S // 2, "last": p.W * p.S - 1}[where]
    p.out[i] ^= 1
    with pytest.raises(AssertionError, match="output byte %d" % i):
        p.check("planted")


@pytest.mark.parametrize("side", ["prefix", "suffix"])
def test_touched_guard_fails(side):
    p, payloads = _gather()
    _write_correct(p, payloads)
    start = wl.GUARD + p.out_off
    i = start - 1 if side == "prefix" else start + p.W * p.S
    p.out_dev[i] = 0
    with pytest.raises(AssertionError, match="%s guard" % side):
        p.check("planted")


def test_far_guard_byte_fails():
    p, payloads = _gather()
    _write_correct(p, payloads)
    p.out_dev[0] = 0
    with pytest.raises(AssertionError, match="prefix guard"):
        p.check("planted")


@pytest.mark.parametrize("r", [0, 2])
def test_changed_source_fails(r):
    p, payloads = _gather()
    _write_correct(p, payloads)
    p.src_dev[r][wl.GUARD + p.in_offs[r] + 4] ^= 0x40
    with pytest.raises(AssertionError, match="source buffer %d changed" % r):
        p.check("planted")


def test_changed_source_guard_fails():
    p, payloads = _gather()
    _write_correct(p, payloads)
    p.src_dev[1][-1] = 0
    with pytest.raises(AssertionError, match="source buffer 1 changed"):
        p.check("planted")


def test_swapped_ranks_fail():
    p, payloads = _gather()
    p.out.copy_(torch.from_numpy(np.concatenate(payloads[::-1])))
    with pytest.raises(AssertionError):
        p.check("planted")


def test_one_wrong_tensor_of_a_batch_fails():
    rng = np.random.default_rng(3)
    payloads = [[rng.integers(0, 256, S, dtype=np.uint8) for _ in range(2)] for S in (5, 64, 300)]
    b = gc.PlacedBatch(2, payloads, [0, 1, 3], [1, 0, 8], CPU)
    for it, pl in zip(b.items, payloads):
        _write_correct(it, pl)
    for t, it in enumerate(b.items):
        it.check("tensor %d" % t)
    b.items[1].out[63] ^= 0xFF
    with pytest.raises(AssertionError, match="output byte 63"):
        b.items[1].check("planted")


# ---------------------------------------------------------------------------
# Rank-ordered sums
# ---------------------------------------------------------------------------

def _bf16(vals):
    return (np.asarray(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _reduce(dtype="bf16", in_place=-1, out_off=3):
    # Element 0: inf + (-inf) = NaN; element 1: 1 + 2^-8 + 2^-8 (an exact
    # bf16 sum); the rest random uniform values.
    rng = np.random.default_rng(5)
    n = 41
    xs = [rng.uniform(-1, 1, n).astype(np.float32) for _ in range(3)]
    xs[0][0], xs[1][0], xs[2][0] = np.inf, -np.inf, 1.0
    xs[0][1], xs[1][1], xs[2][1] = 1.0, 2.0 ** -8, 2.0 ** -8
    if dtype == "bf16":
        payloads = [_bf16(x) for x in xs]
    elif dtype == "f16":
        payloads = [x.astype(np.float16).view(np.uint16) for x in xs]
    else:
        payloads = xs
    return gc.PlacedReduce(payloads, [1, 0, 2], out_off, dtype, CPU, in_place=in_place)


def _write_sum(p):
    p.out.view(torch.uint8).copy_(torch.from_numpy(p.expected().view(np.uint8).copy()))


def _bits(p):
    return p.out.view(torch.int32 if p.es == 4 else torch.int16)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_correct_sum_passes(dtype):
    p = _reduce(dtype)
    _write_sum(p)
    p.check("correct")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_sum_one_ulp_off_fails(dtype):
    p = _reduce(dtype)
    _write_sum(p)
    _bits(p)[5] += 1
    with pytest.raises(AssertionError, match="first 5"):
        p.check("planted")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_finite_where_nan_expected_fails(dtype):
    p = _reduce(dtype)
    _write_sum(p)
    e = p.expected()
    nan0 = {"f32": lambda: np.isnan(e[0]),
            "bf16": lambda: (int(e[0]) & 0x7FFF) > 0x7F80,
            "f16": lambda: (int(e[0]) & 0x7FFF) > 0x7C00}[dtype]()
    assert nan0, "element 0 of the fixture must sum to a NaN"

    _bits(p)[0] = 0
    with pytest.raises(AssertionError, match="first 0"):
        p.check("planted")


def test_nan_where_finite_expected_fails():
    p = _reduce("bf16")
    _write_sum(p)
    _bits(p)[1] = 0x7FC0
    with pytest.raises(AssertionError, match="first 1"):
        p.check("planted")


def test_other_nan_payload_passes():
    # NaN payloads are not specified: any NaN matches a NaN.
    p = _reduce("bf16")
    _write_sum(p)
    _bits(p)[0] = 0x7F81 if int(_bits(p)[0]) != 0x7F81 else 0x7FC0
    p.check("other NaN")


@pytest.mark.parametrize("side", [-1, 1])
def test_sum_guard_fails(side):
    p = _reduce("bf16")
    _write_sum(p)
    nb = p.n * p.es
    p.out_dev[p.out_start - 1 if side < 0 else p.out_start + nb] = 0
    with pytest.raises(AssertionError, match="guard byte changed"):
        p.check("planted")


def test_sum_changed_source_fails():
    p = _reduce("bf16")
    _write_sum(p)
    p.src_dev[2][wl.GUARD + 2 * p.es + 1] ^= 1
    with pytest.raises(AssertionError, match="source buffer 2 changed"):
        p.check("planted")


def test_in_place_sum_passes_and_catches_writes_past_its_output():
    p = _reduce("bf16", in_place=1)
    p.reset()
    _write_sum(p)
    p.check("in place")
    nb = p.n * p.es
    p.out_dev[p.out_start + nb] ^= 1        # one byte past the in-place output
    with pytest.raises(AssertionError, match="guard byte changed"):
        p.check("planted")
    p.reset()
    _write_sum(p)
    p.out_dev[p.out_start - 1] ^= 1         # one byte before it
    with pytest.raises(AssertionError, match="guard byte changed"):
        p.check("planted")


def test_expected_is_the_oracle():
    p = _reduce("f32")
    want = np.empty(p.n, np.float32)
    oracle.reduce_c(p.payloads, want, "f32")
    assert np.array_equal(want.view(np.uint32), p.expected().view(np.uint32))
