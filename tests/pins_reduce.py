"""Pins for the rank-ordered sum: checks fixed by the reading of the pages and
by IEEE-754 arithmetic, independent of any implementation under test.

A ``reduce`` under test has the signature ``reduce(srcs, dtype) -> array``:
``srcs`` are W equal-length 1-D arrays (float32 for "f32", uint16 bf16 /
binary16 bit patterns for "bf16" / "f16"); it returns the n results in the
same storage type.

The reading (the pages -- RL-Align/RL-Kernel PR #491, "Not in this PR" -- name
deterministic all_reduce / reduce_scatter but print no arithmetic): the sum is
taken in rank order, ((x_0 + x_1) + x_2) + ..., every addition a binary32
addition rounded to nearest-even, bf16 inputs widened exactly, the first term
taken as it is, and the result rounded once to the element type
(nearest-even).  What each pin rests on:

* integer sums -- with integer inputs whose partial sums stay exact, every
  order and precision gives the exact integer sum (closed form);
* rank order -- inputs around 2^24 whose binary32 sum depends on the order;
  the values follow by hand from round-to-nearest-even;
* binary32 accumulation -- inputs whose sum differs when accumulated in
  binary64, or rounded to bf16 after every addition;
* error bound -- the binary32 recursive-summation bound (Higham, "Accuracy and
  Stability of Numerical Algorithms", 2nd ed., section 4.2) against the exact
  sum (math.fsum), plus half a bf16 ulp for the final rounding;
* identity -- W = 1 returns its input (every non-NaN bf16 pattern);
* special values -- infinities, NaN, signed zeros, overflow, subnormals, by
  IEEE-754 rules;
* bf16 rounding -- torch's CPU float32 -> bfloat16 conversion (a library
  routine, round to nearest-even) and hand-worked ties;
* binary16 -- the same integer, order, accumulation and special-value pins
  worked for binary16, the identity over every pattern, pairs against numpy's
  binary16 conversions, and the rounding against numpy's and torch's CPU
  float32 -> float16 conversions and hand-worked ties (overflow at 65520,
  gradual underflow).
"""
from __future__ import annotations

import math
import struct

import numpy as np

U32 = 2.0 ** -24          # binary32 unit roundoff


def f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def f32_from_bits(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def bits_of_f32(x) -> int:
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def bf16_to_float(h: int) -> float:
    return f32_from_bits((int(h) & 0xFFFF) << 16)


def bf16_of_exact(x: float) -> int:
    """bf16 bits of a value known to be exactly representable in bf16."""
    u = bits_of_f32(x)
    assert u & 0xFFFF == 0, x
    return u >> 16


def as_f32(xs):
    return np.array(xs, dtype=np.float32)


def as_bf16(hs):
    return np.array(hs, dtype=np.uint16)


def same_bits(got: np.ndarray, want: np.ndarray, dtype: str) -> bool:
    """Bit equality, except that a NaN matches any NaN (payloads unspecified)."""
    got = np.asarray(got)
    want = np.asarray(want)
    if got.shape != want.shape:
        return False
    if dtype == "f32":
        g, w = got.astype(np.float32), want.astype(np.float32)
        gn, wn = np.isnan(g), np.isnan(w)
        return bool(np.array_equal(gn, wn) and np.array_equal(g.view(np.uint32)[~gn], w.view(np.uint32)[~wn]))
    inf = 0x7F80 if dtype == "bf16" else 0x7C00
    g, w = got.astype(np.uint16), want.astype(np.uint16)
    gn = ((g & 0x7FFF) > inf)
    wn = ((w & 0x7FFF) > inf)
    return bool(np.array_equal(gn, wn) and np.array_equal(g[~gn], w[~wn]))


# ---------------------------------------------------------------------------
# binary16 pins
# ---------------------------------------------------------------------------

def f16_of_exact(x: float) -> int:
    """binary16 bits of a value known to be exactly representable in binary16."""
    h = int(np.array([x], np.float16).view(np.uint16)[0])
    assert float(np.array([h], np.uint16).view(np.float16)[0]) == x, x
    return h


def pin_f16_sums(reduce):
    """Integer sums, rank order, binary32 accumulation and special values for
    binary16 elements (worked by hand)."""
    rng = np.random.default_rng(13)
    for W in (1, 2, 8, 16):
        y = rng.integers(-8, 9, size=(W, 129))
        hs = [np.array([f16_of_exact(float(v)) for v in row], np.uint16) for row in y]
        want = np.array([f16_of_exact(float(v)) for v in y.sum(axis=0)], np.uint16)
        assert np.array_equal(reduce(hs, "f16"), want), W
    # rank order: 2^15 + 2^-9 is a binary32 tie (ulp 2^-8) and rounds to the even
    # 2^15; - 2^15 then gives 0.  Reversed: -2^15 + 2^-9 is exact, + 2^15 = 2^-9.
    big, small = 2.0 ** 15, 2.0 ** -9
    for xs, want in (([big, small, -big], 0.0), ([-big, small, big], small)):
        got = reduce([np.array([f16_of_exact(v)], np.uint16) for v in xs], "f16")
        assert got[0] == f16_of_exact(want), (xs, hex(int(got[0])))
    # binary32 accumulation: 1 + 2^-11 + 2^-11 = 1 + 2^-10 exactly (0x3C01); rounding
    # to binary16 after every add would give 1 + 2^-11 -> 1 (tie, even), twice: 0x3C00
    got = reduce([np.array([h], np.uint16) for h in (0x3C00, f16_of_exact(2.0 ** -11), f16_of_exact(2.0 ** -11))],
                 "f16")
    assert got[0] == 0x3C01
    cases = [
        ([0x7C00, 0x3C00], 0x7C00),               # +inf + 1
        ([0x7C00, 0xFC00], None),                 # +inf + -inf = NaN
        ([0x7E00, 0x3C00], None),                 # NaN + 1
        ([0x7BFF, 0x7BFF], 0x7C00),               # 65504 + 65504 overflows binary16
        ([0x7BFF, f16_of_exact(16.0)], 0x7C00),   # 65520: a tie above 65504 (odd): up to +inf
        ([0x7BFF, f16_of_exact(8.0)], 0x7BFF),    # 65512: below the tie, stays 65504
        ([0x0001, 0x0001], 0x0002),               # subnormals add exactly
        ([0x8001, 0x0001], 0x0000),               # x + (-x) = +0
        ([0x8000, 0x8000], 0x8000),               # -0 + -0 = -0
        ([0x3C00, f16_of_exact(2.0 ** -11)], 0x3C00),      # 1 + 2^-11: tie, to even (1)
        ([0x3C01, f16_of_exact(2.0 ** -11)], 0x3C02),      # (1 + 2^-10) + 2^-11: tie, to even
        ([0x0400, 0x8001], 0x03FF),               # smallest normal - smallest subnormal
    ]
    for hs, want in cases:
        got = reduce([np.array([h], np.uint16) for h in hs], "f16")
        if want is None:
            assert (got[0] & 0x7FFF) > 0x7C00, (hs, hex(int(got[0])))
        else:
            assert got[0] == want, (hs, hex(int(got[0])), hex(want))
    # W = 1 is the identity on every binary16 pattern (NaNs by class)
    every = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    assert same_bits(reduce([every.copy()], "f16"), every, "f16")
    # pairs against numpy's own binary16 widening and binary32 -> binary16
    # rounding (library routines): x + y in binary32, rounded once
    bits = rng.integers(0, 1 << 16, size=(2, 20000), dtype=np.uint32).astype(np.uint16)
    with np.errstate(over="ignore", invalid="ignore"):
        want = (bits[0].view(np.float16).astype(np.float32) + bits[1].view(np.float16).astype(np.float32))
        want = want.astype(np.float16).view(np.uint16)
    assert same_bits(reduce([bits[0].copy(), bits[1].copy()], "f16"), want, "f16")


def pin_f16_rounding(round_fn):
    """``round_fn(float32 array) -> uint16 binary16 bits`` against hand-worked
    ties and numpy's and torch's CPU conversions."""
    import torch
    hand = {0x3F801000: 0x3C00,     # 1 + 2^-11: tie, even stays
            0x3F803000: 0x3C02,     # 1 + 3*2^-11: tie, odd rounds up
            0x3F801001: 0x3C01,     # just above the tie
            0x477FE000: 0x7BFF,     # 65504, the largest binary16, exactly
            0x477FE800: 0x7BFF,     # 65512: below the tie, down to 65504
            0x477FF000: 0x7C00,     # 65520: the tie above 65504 (odd) -> +inf
            0x477FEFFF: 0x7BFF,     # just below 65520
            0x477FF800: 0x7C00,     # 65528: above the tie -> +inf
            0x33000000: 0x0000,     # 2^-25: tie with 0 and 2^-24, to even (0)
            0x33400000: 0x0001,     # 1.5 * 2^-25 -> 2^-24
            0x33C00000: 0x0002,     # 3 * 2^-25: tie, to even (2 * 2^-24)
            0x387FE000: 0x0400,     # 2^-14 - 2^-25: tie between 0x03FF (odd) and 0x0400
            0x7F800000: 0x7C00, 0xFF800000: 0xFC00, 0x80000000: 0x8000, 0x00000001: 0x0000}
    xs = np.array(list(hand), dtype=np.uint32).view(np.float32)
    got = np.asarray(round_fn(xs))
    for k, (u, want) in enumerate(hand.items()):
        assert got[k] == want, (hex(u), hex(int(got[k])), hex(want))
    rng = np.random.default_rng(19)
    bits = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    bits[:5000] = (bits[:5000] & 0xFFFFE000) | 0x1000          # ties at the normal quantum
    bits[5000:6000] = (bits[5000:6000] & 0x807FFFFF) | (np.uint32(100) << 23)   # subnormal range
    xs = bits.view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        want_np = xs.astype(np.float16).view(np.uint16)
    want_t = torch.from_numpy(xs.copy()).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    got = np.asarray(round_fn(xs))
    assert same_bits(got, want_np, "f16")
    assert same_bits(got, want_t, "f16")


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def pin_integer_sums(reduce):
    rng = np.random.default_rng(5)
    for W in (1, 2, 3, 8, 16):
        # binary32: |x| <= 2^20, W <= 16: every partial sum is an integer below 2^24
        x = rng.integers(-(1 << 20), (1 << 20) + 1, size=(W, 257))
        got = reduce([as_f32(r) for r in x], "f32")
        assert np.array_equal(got, x.sum(axis=0).astype(np.float32)), W
        # bf16: |x| <= 8, W <= 16: the sum is an integer of at most 8 bits, exact in bf16
        y = rng.integers(-8, 9, size=(W, 257))
        hs = [as_bf16([bf16_of_exact(float(v)) for v in row]) for row in y]
        want = as_bf16([bf16_of_exact(float(v)) for v in y.sum(axis=0)])
        assert np.array_equal(reduce(hs, "bf16"), want), W


def pin_rank_order(reduce):
    big = float(1 << 24)
    # 2^24 + 1 is a tie between 2^24 and 2^24 + 2 and rounds to the even 2^24;
    # then - 2^24 leaves 0.  Any order that meets -2^24 before 2^24 gives 1.
    cases = [([big, 1.0, -big], 0.0),
             # rank order: 1 + 2^24 -> 2^24 (tie), + 1 -> 2^24 (tie), - 2^24 -> 0,
             # + 1 -> 1.  The exact sum, and the reversed order, give 3.
             ([1.0, big, 1.0, -big, 1.0], 1.0),
             # -2^24 + 1 = -16777215 and 1 - 2^24 are exact; + 2^24 then gives 1
             ([-big, 1.0, big], 1.0),
             ([1.0, -big, big], 1.0)]
    for xs, want in cases:
        srcs = [as_f32([v]) for v in xs]
        assert reduce(srcs, "f32")[0] == np.float32(want), (xs, want)
        hs = [as_bf16([bf16_of_exact(v)]) for v in xs]
        assert reduce(hs, "bf16")[0] == bf16_of_exact(want), (xs, want)
    # Position matters element by element: the same triple rotated across
    # elements gives each element its own order.
    trip = [big, 1.0, -big]
    srcs = [as_f32([trip[(r + k) % 3] for k in range(3)]) for r in range(3)]
    # element k sums trip[k], trip[k+1], trip[k+2] (indices mod 3) in rank order:
    # [2^24, 1, -2^24] -> 0;  [1, -2^24, 2^24] -> 1;  [-2^24, 2^24, 1] -> 1
    assert np.array_equal(reduce(srcs, "f32"), as_f32([0.0, 1.0, 1.0]))


def pin_binary32_accumulation(reduce):
    # binary32: 1 + 2^-24 is a tie and rounds to 1; twice more stays 1.  In
    # binary64 the sum would be 1 + 2^-23 (a binary32 number).
    srcs = [as_f32([1.0]), as_f32([2.0 ** -24]), as_f32([2.0 ** -24])]
    assert reduce(srcs, "f32")[0] == np.float32(1.0)
    # bf16 inputs, binary32 accumulation: 1 + 2^-8 + 2^-8 = 1 + 2^-7 exactly,
    # which bf16 holds (0x3F81).  Rounding to bf16 after every addition would
    # give 1 + 2^-8 -> 1 (tie to even), twice: 0x3F80.
    hs = [as_bf16([0x3F80]), as_bf16([bf16_of_exact(2.0 ** -8)]), as_bf16([bf16_of_exact(2.0 ** -8)])]
    assert reduce(hs, "bf16")[0] == 0x3F81


def pin_error_bound(reduce):
    rng = np.random.default_rng(11)
    for W in (2, 3, 8, 33):
        x = (rng.random((W, 300), dtype=np.float32) * 2 - 1) * np.float32(1000)
        got = reduce([r.copy() for r in x], "f32").astype(np.float64)
        gamma = (W - 1) * U32 / (1 - (W - 1) * U32)
        for i in range(x.shape[1]):
            col = [float(v) for v in x[:, i]]
            exact = math.fsum(col)
            bound = gamma * math.fsum(abs(v) for v in col)
            assert abs(got[i] - exact) <= bound * (1 + 1e-12) + 1e-300, (W, i, got[i], exact, bound)
        hs = []
        for r in range(W):
            v = x[r] / np.float32(1000)
            hs.append(as_bf16([(bits_of_f32(f32(float(a))) >> 16) for a in v]))
        gotb = reduce(hs, "bf16")
        for i in range(x.shape[1]):
            col = [bf16_to_float(h[i]) for h in hs]
            exact = math.fsum(col)
            bound = gamma * math.fsum(abs(v) for v in col)
            s32 = abs(exact) + bound
            # final rounding to bf16: half an ulp, at most 2^-8 relative
            total = bound + s32 * 2.0 ** -8 + 2.0 ** -133
            assert abs(bf16_to_float(gotb[i]) - exact) <= total, (W, i)


def pin_identity(reduce):
    every = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = reduce([every.copy()], "bf16")
    assert same_bits(got, every, "bf16")
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 32, size=4096, dtype=np.uint64).astype(np.uint32)
    xs = bits.view(np.float32)
    assert same_bits(reduce([xs.copy()], "f32"), xs, "f32")


def pin_special_values(reduce):
    inf, nan = float("inf"), float("nan")
    fmax = f32_from_bits(0x7F7FFFFF)
    tiny = f32_from_bits(0x00000001)              # 2^-149, smallest subnormal
    cases_f32 = [
        ([inf, 1.0], inf), ([-inf, 1.0], -inf), ([inf, -inf], nan), ([nan, 1.0], nan),
        ([1.0, nan], nan), ([fmax, fmax], inf), ([fmax, -fmax], 0.0),
        ([tiny, tiny], f32_from_bits(2)), ([f32_from_bits(0x00800000), -tiny], f32_from_bits(0x007FFFFF)),
        ([1.0, -1.0], 0.0),
    ]
    for xs, want in cases_f32:
        got = reduce([as_f32([v]) for v in xs], "f32")
        assert same_bits(got, as_f32([want]), "f32"), (xs, got, want)
    # signed zeros: -0 + -0 = -0; +0 + -0 = +0 (round to nearest); a lone -0 stays -0
    for xs, sign in (([-0.0, -0.0], 1), ([0.0, -0.0], 0), ([-0.0, 0.0], 0), ([-0.0], 1), ([-0.0, -0.0, -0.0], 1)):
        got = reduce([as_f32([v]) for v in xs], "f32")
        assert got.view(np.uint32)[0] == (0x80000000 if sign else 0), xs
        hb = reduce([as_bf16([0x8000 if math.copysign(1, v) < 0 else 0]) for v in xs], "bf16")
        assert hb[0] == (0x8000 if sign else 0), xs
    cases_bf16 = [
        ([0x7F80, 0x3F80], 0x7F80),                 # +inf + 1
        ([0x7F80, 0xFF80], None),                   # +inf + -inf = NaN
        ([0x7FC0, 0x3F80], None),                   # NaN + 1 = NaN
        ([0x7F7F, 0x7F7F], 0x7F80),                 # overflow in binary32
        # 0x7F7F = (2 - 2^-7) 2^127; + 2^119 gives (2 - 2^-8) 2^127, exact in
        # binary32 and a bf16 tie between 0x7F7F (odd) and 2^128: rounds up to +inf
        ([0x7F7F, bf16_of_exact(2.0 ** 119)], 0x7F80),
        ([0x0001, 0x0001], 0x0002),                 # subnormals add exactly
        ([0x8001, 0x0001], 0x0000),                 # x + (-x) = +0
        ([0x3F80, 0x3B80], 0x3F80),                 # 1 + 2^-8: tie, to even (1)
        ([0x3F81, 0x3B80], 0x3F82),                 # (1 + 2^-7) + 2^-8: tie, to even (1 + 2^-6)
    ]
    for hs, want in cases_bf16:
        got = reduce([as_bf16([h]) for h in hs], "bf16")
        if want is None:
            assert (got[0] & 0x7FFF) > 0x7F80, (hs, hex(got[0]))
        else:
            assert got[0] == want, (hs, hex(got[0]), hex(want))


def pin_bf16_rounding(round_fn):
    """``round_fn(float32 array) -> uint16 bf16 bits`` against hand-worked ties
    and torch's CPU conversion."""
    import torch
    hand = {0x3F808000: 0x3F80,     # 1 + 2^-8: tie, even stays
            0x3F818000: 0x3F82,     # 1 + 2^-7 + 2^-8: tie, odd rounds up
            0x3F808001: 0x3F81,     # just above the tie
            0x3F807FFF: 0x3F80,     # just below
            0xBF808000: 0xBF80,     # negative tie
            0x7F7FFFFF: 0x7F80,     # rounds up to +inf
            0x00008000: 0x0000,     # subnormal tie, even
            0x00018000: 0x0002,     # subnormal tie, odd up
            0x7F800000: 0x7F80, 0xFF800000: 0xFF80, 0x80000000: 0x8000}
    xs = np.array(list(hand), dtype=np.uint32).view(np.float32)
    got = np.asarray(round_fn(xs))
    for k, (u, want) in enumerate(hand.items()):
        assert got[k] == want, (hex(u), hex(int(got[k])), hex(want))
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties and near-ties
    bits[:5000] = (bits[:5000] & 0xFFFF0000) | 0x8000
    bits[5000:6000] = (bits[5000:6000] & 0xFFFF0000) | 0x7FFF
    bits[6000:7000] = (bits[6000:7000] & 0xFFFF0000) | 0x8001
    xs = bits.view(np.float32)
    want = torch.from_numpy(xs.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert same_bits(np.asarray(round_fn(xs)), want, "bf16")
