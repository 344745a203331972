"""The rank-ordered-sum oracle against its pins (CPU only).

The C oracle and the pure-Python oracle each pass every pin in
``tests/pins_reduce.py``, agree with each other bit for bit on seeded inputs,
and every planted mistake below (a plausible slip in a deterministic sum)
fails at least one pin.
"""
from __future__ import annotations

import numpy as np
import pytest

from deterministic_collective_movement_amd import workloads as wl
from oracle import oracle
from tests import pins_reduce as pins


def c_reduce(srcs, dtype):
    out = np.empty(srcs[0].shape[0], dtype=oracle.REDUCE_DTYPES[dtype])
    return oracle.reduce_c([np.ascontiguousarray(s) for s in srcs], out, dtype)


def py_reduce(srcs, dtype):
    if dtype == "f32":
        return np.array(oracle.reduce_py([s.tolist() for s in srcs], "f32"), dtype=np.float32)
    return np.array(oracle.reduce_py([[int(v) for v in s] for s in srcs], dtype), dtype=np.uint16)


ORACLES = {"c": c_reduce, "py": py_reduce}
PINS = [pins.pin_integer_sums, pins.pin_rank_order, pins.pin_binary32_accumulation,
        pins.pin_error_bound, pins.pin_special_values]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
@pytest.mark.parametrize("which", sorted(ORACLES))
def test_oracle_passes_pin(which, pin):
    pin(ORACLES[which])


def test_c_oracle_identity():
    pins.pin_identity(c_reduce)


def test_bf16_rounding_of_both_oracles():
    pins.pin_bf16_rounding(oracle.f32_to_bf16_c)
    pins.pin_bf16_rounding(lambda xs: np.array([oracle.f32_to_bf16_py(float(v)) for v in xs], np.uint16))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [1, 2, 3, 7, 8])
def test_c_and_python_oracles_agree(dtype, W):
    """Seeded inputs from the shared generators, including random bit patterns
    (NaNs, infinities, subnormals): the two oracles agree bit for bit."""
    for kind in ("uniform", "bits"):
        srcs = wl.reduce_payloads(wl.case_seed(7, W), W, 97, dtype, kind)
        assert pins.same_bits(c_reduce(srcs, dtype), py_reduce(srcs, dtype), dtype), (dtype, W, kind)


# ---------------------------------------------------------------------------
# Planted mistakes: each must fail a pin
# ---------------------------------------------------------------------------

def _widen(srcs, dtype):
    if dtype == "f32":
        return [s.astype(np.float32) for s in srcs]
    return [(s.astype(np.uint32) << 16).view(np.float32) for s in srcs]


def _narrow(acc, dtype):
    if dtype == "f32":
        return acc.astype(np.float32)
    return oracle.f32_to_bf16_c(acc)


def _mistake(order=None, accum=np.float32, step_round=False, init_zero=False, drop_last=False,
             truncate=False, negate_last=False):
    def reduce(srcs, dtype):
        with np.errstate(over="ignore", invalid="ignore"):
            return _run(srcs, dtype)

    def _run(srcs, dtype):
        xs = _widen(srcs, dtype)
        if drop_last and len(xs) > 1:
            xs = xs[:-1]
        if negate_last and len(xs) > 1:
            xs = xs[:-1] + [-xs[-1]]
        if order == "reverse":
            xs = xs[::-1]
        acc = np.zeros_like(xs[0], dtype=accum) if init_zero else xs[0].astype(accum)
        for x in (xs if init_zero else xs[1:]):
            acc = (acc + x.astype(accum)).astype(accum)
            if step_round and dtype == "bf16":
                acc = _widen([oracle.f32_to_bf16_c(acc.astype(np.float32))], "bf16")[0].astype(accum)
        acc = acc.astype(np.float32)
        if truncate and dtype == "bf16":
            return (acc.view(np.uint32) >> 16).astype(np.uint16)
        return _narrow(acc, dtype)
    return reduce


MISTAKES = {
    "reversed_ranks": _mistake(order="reverse"),
    "binary64_accumulation": _mistake(accum=np.float64),
    "bf16_after_every_add": _mistake(step_round=True),
    "zero_initialised": _mistake(init_zero=True),
    "last_rank_dropped": _mistake(drop_last=True),
    "truncating_bf16": _mistake(truncate=True),
    "last_rank_subtracted": _mistake(negate_last=True),
}


def _fails_some_pin(reduce):
    for pin in PINS + [pins.pin_identity]:
        try:
            pin(reduce)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistake_is_caught(name):
    assert _fails_some_pin(MISTAKES[name]), name


def test_the_mistake_harness_itself_passes_when_correct():
    correct = _mistake()
    for pin in PINS + [pins.pin_identity]:
        pin(correct)


# ---------------------------------------------------------------------------
# binary16
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("which", sorted(ORACLES))
def test_oracle_passes_f16_pins(which):
    pins.pin_f16_sums(ORACLES[which])


def test_f16_rounding_of_both_oracles():
    pins.pin_f16_rounding(oracle.f32_to_f16_c)
    pins.pin_f16_rounding(lambda xs: np.array([oracle.f32_to_f16_py(float(v)) for v in xs], np.uint16))


@pytest.mark.parametrize("W", [1, 2, 5, 8])
def test_c_and_python_oracles_agree_f16(W):
    for kind in ("uniform", "bits"):
        srcs = wl.reduce_payloads(wl.case_seed(8, W), W, 97, "f16", kind)
        assert pins.same_bits(c_reduce(srcs, "f16"), py_reduce(srcs, "f16"), "f16"), (W, kind)
