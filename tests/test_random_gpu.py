"""Seeded random cases on the GPU: gathers and rank-ordered sums with random W,
sizes (spread over six decades), byte / element offsets, element types and
forced paths, each checked against the CPU oracle (every byte and every guard
for gathers; every element, NaN by class, for sums).  The seed list is fixed,
so a failure names a reproducible case."""
from __future__ import annotations

import numpy as np
import pytest

from deterministic_collective_movement_amd import workloads as wl
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

N_CASES = 120


def _size(rng, lo_exp, hi_exp):
    return int(10 ** rng.uniform(lo_exp, hi_exp))


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_gather(gpu, seed):
    rng = np.random.default_rng([4242, seed])
    W = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 13, 64]))
    S = _size(rng, 0, 6.3 if W <= 8 else 4.5)
    in_offs = [int(rng.integers(0, 16)) if rng.random() < 0.5 else 0 for _ in range(W)]
    out_off = int(rng.integers(0, 16)) if rng.random() < 0.5 else 0
    path = int(rng.choice(gc.PATHS))
    payloads = [wl.random_bytes(wl.case_seed(21, seed), r, S) for r in range(W)]
    placed = gc.Placed(payloads, in_offs, out_off, gpu)
    gc.run_all_paths(placed, "random gather #%d W=%d S=%d in=%s out=%d" % (seed, W, S, in_offs, out_off),
                     paths=(path,))


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_sum(gpu, seed):
    rng = np.random.default_rng([4343, seed])
    W = int(rng.choice([1, 2, 3, 4, 6, 8, 11, 32, 64]))
    dtype = str(rng.choice(["bf16", "f16", "f32"]))
    n = _size(rng, 0, 6.0 if W <= 8 else 4.5)
    in_offs = [int(rng.integers(0, 16)) if rng.random() < 0.5 else 0 for _ in range(W)]
    out_off = int(rng.integers(0, 16)) if rng.random() < 0.5 else 0
    kind = "bits" if rng.random() < 0.25 else "uniform"
    path = int(rng.choice(gc.PATHS))
    payloads = wl.reduce_payloads(wl.case_seed(22, seed), W, n, dtype, kind)
    placed = gc.PlacedReduce(payloads, in_offs, out_off, dtype, gpu)
    gc.run_reduce_all_paths(placed, "random sum #%d W=%d n=%d %s %s in=%s out=%d"
                            % (seed, W, n, dtype, kind, in_offs, out_off), paths=(path,))
