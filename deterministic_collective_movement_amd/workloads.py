"""Seeded synthetic inputs for the rank-ordered gather and the rank-ordered sum.

This module generates input bytes and case lists only.  It holds none of the
methods' arithmetic: no concatenation, no output layout, no alignment decision,
no addition and no rounding to bf16 of a sum.
Both the GPU tests and the CPU oracle draw their inputs from here, so both see
the same bytes.

The workloads follow the pages' measurements: RL-Align/RL-Kernel PR #491
("Results", B200 and H100 tables: BF16 payloads of 1 KiB .. 4 MiB per rank at
2, 4 and 8 ranks, median of 100 calls) and its size test ("Tests": byte sizes
on both sides of the one-block bound, sizes that end off a 16-byte boundary,
and sources and outputs at byte offsets).
The batched mix borrows the 8627 x 8192 BF16 activation shape of
vllm-project/vllm PR #57037 ("[Benchmark] Add all-reduce rank-skew
calibration", the reproduction command and its results table).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

KiB = 1024
MiB = 1024 * KiB

#: Guard bytes around every carved buffer, and their sentinel value.  The
#: pages' size test fills the storage with 0xA5 and keeps a 16-byte tail guard
#: (PR #491 review threads on the size test); 64 bytes each side is our choice.
GUARD = 64
GUARD_BYTE = 0xA5

#: Offsets swept by the alignment test (the pages test four input/output
#: offsets without printing them; these four mix odd, 4-aligned and 8-aligned).
OFFSETS = (0, 1, 3, 8)


def case_seed(config: int, case_index: int) -> int:
    """Per-case seed: 1_000_003 * config + case_index."""
    return 1_000_003 * config + case_index


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def random_bytes(seed: int, stream: int, nbytes: int) -> np.ndarray:
    """nbytes uniformly random bytes (uint8), reproducible from (seed, stream)."""
    return np.frombuffer(_rng(seed, stream).bytes(nbytes), dtype=np.uint8).copy()


def bf16_random_bits(seed: int, stream: int, n_elems: int) -> np.ndarray:
    """n_elems bf16 values with uniformly random 16-bit patterns, as 2*n_elems bytes.

    Random patterns include NaNs, so results are always compared as bytes.
    """
    return random_bytes(seed, stream, 2 * n_elems)


def bf16_uniform(seed: int, stream: int, n_elems: int) -> np.ndarray:
    """n_elems bf16 values uniform in [-1, 1] as bytes: float32 draws cut to their
    top 16 bits (rounded toward zero; no rounding of either method here)."""
    rng = _rng(seed, stream)
    out = np.empty(n_elems, dtype=np.uint16)
    step = 1 << 24
    for lo in range(0, n_elems, step):
        hi = min(n_elems, lo + step)
        f = rng.random(hi - lo, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
        out[lo:hi] = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return out.view(np.uint8)


def tagged_payload(r: int, nbytes: int) -> np.ndarray:
    """Peer-tagged bytes: byte i of payload r is (r*131 + i*7 + 1) mod 251.

    Any misrouted byte (wrong peer, wrong offset, off by one) changes the value.
    """
    i = np.arange(nbytes, dtype=np.int64)
    return ((r * 131 + i * 7 + 1) % 251).astype(np.uint8)


# ---------------------------------------------------------------------------
# Case lists
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class GatherCase:
    """One gather: W payloads of S bytes; payload r starts at in_offs[r] bytes
    into its own guarded buffer, the output at out_off bytes into its buffer."""
    config: int
    index: int
    W: int
    S: int
    in_offs: Tuple[int, ...]
    out_off: int
    kind: str = "bytes"          # "bytes", "bf16_bits" or "bf16_uniform"

    @property
    def seed(self) -> int:
        return case_seed(self.config, self.index)

    def payload(self, r: int) -> np.ndarray:
        if self.kind == "bf16_uniform":
            assert self.S % 2 == 0
            return bf16_uniform(self.seed, r, self.S // 2)
        if self.kind == "bf16_bits":
            assert self.S % 2 == 0
            return bf16_random_bits(self.seed, r, self.S // 2)
        return random_bytes(self.seed, r, self.S)

    def label(self) -> str:
        offs = ",".join(str(o) for o in self.in_offs)
        return f"c{self.config}#{self.index}:W={self.W},S={self.S},in=[{offs}],out={self.out_off}"


def config1() -> List[GatherCase]:
    """W=2 payloads of 1 KiB (512 bf16 random bit patterns), all 16-byte aligned."""
    return [GatherCase(1, 0, 2, 1 * KiB, (0, 0), 0, "bf16_bits")]


CONFIG2_W = (2, 8)
CONFIG2_S = (1 * KiB, 8 * KiB, 32 * KiB, 128 * KiB, 1 * MiB, 4 * MiB)


def config2() -> List[GatherCase]:
    """Size sweep of the pages' tables: W in {2, 8} x S in {1,8,32,128 KiB, 1,4 MiB}, aligned."""
    cases = []
    for W in CONFIG2_W:
        for S in CONFIG2_S:
            cases.append(GatherCase(2, len(cases), W, S, (0,) * W, 0, "bf16_bits"))
    return cases


CONFIG3_W = (2, 3, 8)
CONFIG3_S = (1, 15, 17, 4095, 64 * KiB - 1, 64 * KiB, 64 * KiB + 1, 256 * KiB + 7)


def config3() -> List[GatherCase]:
    """Alignment/tail sweep: W x S x in_off (all peers) x out_off = 384 cases, plus one
    mixed case per (W, S) with peer r at offset OFFSETS[r % 4]."""
    cases = []
    for W in CONFIG3_W:
        for S in CONFIG3_S:
            for io in OFFSETS:
                for oo in OFFSETS:
                    cases.append(GatherCase(3, len(cases), W, S, (io,) * W, oo))
    for W in CONFIG3_W:
        for S in CONFIG3_S:
            offs = tuple(OFFSETS[r % 4] for r in range(W))
            cases.append(GatherCase(3, len(cases), W, S, offs, 0))
    return cases


def config4() -> GatherCase:
    """Bandwidth regime: W=8 aligned bf16 payloads of 64 MiB (uniform in [-1, 1])."""
    return GatherCase(4, 0, 8, 64 * MiB, (0,) * 8, 0, "bf16_uniform")


@dataclass(frozen=True)
class BatchTensor:
    rows: int
    cols: int
    in_off: int
    out_off: int

    @property
    def S(self) -> int:
        return self.rows * self.cols * 2


@dataclass(frozen=True)
class BatchCase:
    config: int
    index: int
    W: int
    tensors: Tuple[BatchTensor, ...] = field(default_factory=tuple)

    @property
    def seed(self) -> int:
        return case_seed(self.config, self.index)

    def payload(self, t: int, r: int) -> np.ndarray:
        return bf16_random_bits(self.seed, t * self.W + r, self.tensors[t].S // 2)

    def total_bytes_moved(self) -> int:
        return sum(2 * self.W * x.S for x in self.tensors)


CONFIG5_COLS = (128, 1024, 8192)
CONFIG5_MAX_ROWS = 8627


def config5(index: int = 0, n: int = 16, W: int = 4, max_rows: int = CONFIG5_MAX_ROWS) -> BatchCase:
    """Batched gather: n tensors of rows ~ U{1..max_rows} x cols ~ U{128,1024,8192} bf16;
    each tensor is odd with probability 1/2, and an odd tensor draws its input and
    output byte offsets independently from {1, 3}; even tensors sit at offset 0."""
    rng = _rng(case_seed(5, index), 1 << 20)
    tensors = []
    for _ in range(n):
        rows = int(rng.integers(1, max_rows + 1))
        cols = int(CONFIG5_COLS[int(rng.integers(0, len(CONFIG5_COLS)))])
        odd = bool(rng.integers(0, 2))
        if odd:
            io = int((1, 3)[int(rng.integers(0, 2))])
            oo = int((1, 3)[int(rng.integers(0, 2))])
        else:
            io = oo = 0
        tensors.append(BatchTensor(rows, cols, io, oo))
    return BatchCase(5, index, W, tuple(tensors))


# ---------------------------------------------------------------------------
# Rank-ordered sum (the reduction of a deterministic all-reduce)
# ---------------------------------------------------------------------------

#: Bytes of one element of each element type of the sum.
REDUCE_ESIZE = {"f32": 4, "bf16": 2, "f16": 2}


def reduce_payloads(seed: int, W: int, n: int, dtype: str, kind: str = "uniform") -> List[np.ndarray]:
    """W payloads of n elements, reproducible from (seed, payload index).

    dtype "f32": float32 arrays; "bf16" / "f16": uint16 arrays of bf16 /
    binary16 bit patterns.
    kind "uniform": values uniform in [-1, 1) (bf16: the float32 draw cut to its
    top 16 bits, i.e. rounded toward zero; f16: a random sign, a random
    significand and an exponent uniform over 2^-14 .. 2^0, i.e. normal
    binary16 values of magnitude below 2, built bit by bit); "bits": uniformly
    random bit patterns (NaNs, infinities and subnormals included).
    """
    out = []
    for r in range(W):
        rng = _rng(seed, r)
        if kind == "bits":
            b = rng.bytes(n * REDUCE_ESIZE[dtype])
            out.append(np.frombuffer(b, np.float32 if dtype == "f32" else np.uint16).copy())
            continue
        if dtype == "f16":
            sign = rng.integers(0, 2, n, dtype=np.uint16) << np.uint16(15)
            expo = rng.integers(1, 16, n, dtype=np.uint16) << np.uint16(10)
            mant = rng.integers(0, 1 << 10, n, dtype=np.uint16)
            out.append((sign | expo | mant).astype(np.uint16))
            continue
        f = rng.random(n, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
        out.append(f if dtype == "f32" else (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16))
    return out


@dataclass(frozen=True)
class ReduceCase:
    """One rank-ordered sum: W payloads of n elements; payload r starts in_offs[r]
    elements into its own guarded buffer, the output out_off elements into its."""
    config: int
    index: int
    W: int
    n: int
    dtype: str
    in_offs: Tuple[int, ...]
    out_off: int
    kind: str = "uniform"

    @property
    def seed(self) -> int:
        return case_seed(self.config, self.index)

    @property
    def esize(self) -> int:
        return REDUCE_ESIZE[self.dtype]

    def payloads(self) -> List[np.ndarray]:
        return reduce_payloads(self.seed, self.W, self.n, self.dtype, self.kind)

    def label(self) -> str:
        offs = ",".join(str(o) for o in self.in_offs)
        return f"r{self.config}#{self.index}:W={self.W},n={self.n},{self.dtype},in=[{offs}],out={self.out_off}"


REDUCE_SWEEP_W = (2, 8)
#: Per-rank bytes of the pages' deterministic collective sweep, across the
#: 256 KiB single-block bound of their all_reduce / reduce_scatter.
REDUCE_SWEEP_BYTES = (1 * KiB, 8 * KiB, 32 * KiB, 128 * KiB, 256 * KiB, 512 * KiB, 1 * MiB, 4 * MiB)


def reduce_config1() -> List[ReduceCase]:
    """W=2 bf16 payloads of 1 KiB (512 elements), aligned."""
    return [ReduceCase(11, 0, 2, 512, "bf16", (0, 0), 0)]


def reduce_config2() -> List[ReduceCase]:
    """Size sweep: W in {2, 8} x per-rank 1 KiB .. 4 MiB of bf16, aligned."""
    cases = []
    for W in REDUCE_SWEEP_W:
        for nb in REDUCE_SWEEP_BYTES:
            cases.append(ReduceCase(12, len(cases), W, nb // 2, "bf16", (0,) * W, 0))
    return cases


REDUCE_TAIL_N = (1, 7, 9, 2047, 32767, 32768, 32769, 131075)
REDUCE_ELEM_OFFSETS = (0, 1, 3, 8)


def reduce_config3() -> List[ReduceCase]:
    """Alignment / tail sweep: bf16, binary16 and binary32 x W in {2, 3, 8} x n x
    element offsets of the sources (all alike) and of the output, plus a
    mixed-offset case per (dtype, W, n) and random-bit-pattern cases."""
    cases = []
    for dtype in ("bf16", "f16", "f32"):
        for W in (2, 3, 8):
            for n in REDUCE_TAIL_N:
                for io in REDUCE_ELEM_OFFSETS:
                    for oo in REDUCE_ELEM_OFFSETS:
                        cases.append(ReduceCase(13, len(cases), W, n, dtype, (io,) * W, oo))
                offs = tuple(REDUCE_ELEM_OFFSETS[r % 4] for r in range(W))
                cases.append(ReduceCase(13, len(cases), W, n, dtype, offs, 1))
                cases.append(ReduceCase(13, len(cases), W, n, dtype, offs, 0, "bits"))
    return cases


def reduce_config4() -> ReduceCase:
    """Bandwidth regime: W=8 aligned bf16 payloads of 64 MiB (32 Mi elements)."""
    return ReduceCase(14, 0, 8, 32 * MiB, "bf16", (0,) * 8, 0)


def carve(total: int, offset: int) -> Tuple[int, int]:
    """Size of a guarded host/device allocation and the data start inside it."""
    return GUARD + offset + total + GUARD, GUARD + offset
