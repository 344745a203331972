"""Seeded random cases on the GPU: gathers and rank-ordered sums with random W,
sizes (spread over six decades), byte / element offsets, element types and
forced paths, each checked against the CPU oracle (every byte and every guard
for gathers; every element, NaN by class, for sums).  The seed list is fixed,
so a failure names a reproducible case."""
from __future__ import annotations

import numpy as np
import pytest

from deterministic_collective_movement_amd import rog
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


N_STREAMED = 12


@pytest.mark.parametrize("seed", range(N_STREAMED))
def test_random_streamed_gather(gpu, seed):
    """Seeded random gathers over 128 - 200 MiB of sources, where loads stream
    past the caches (FLAT with non-temporal loads; PEER with its shuffled
    granule body at odd and 2-mod-4 source offsets): random W, payload size
    and byte offsets, every byte and guard against the oracle."""
    rng = np.random.default_rng([4444, seed])
    W = int(rng.choice([2, 3, 4, 5, 8, 16]))
    total = int(rng.integers((128 << 20) + 4096, 200 << 20))
    S = total // W + int(rng.integers(0, 64))
    in_offs = [int(rng.integers(0, 16)) if rng.random() < 0.5 else 0 for _ in range(W)]
    if rng.random() < 0.3:
        in_offs = [0] * W
    out_off = 0 if all(o == 0 for o in in_offs) and rng.random() < 0.5 else int(rng.integers(0, 16))
    payloads = [wl.random_bytes(wl.case_seed(23, seed), r, S) for r in range(W)]
    placed = gc.Placed(payloads, in_offs, out_off, gpu)
    plan = rog.rog_plan(placed.srcs, placed.out)
    assert plan["nt_loads"]
    gc.run_all_paths(placed, "random streamed gather #%d W=%d S=%d in=%s out=%d" % (seed, W, S, in_offs, out_off),
                     paths=(rog.ROG_PATH_AUTO,))


@pytest.mark.parametrize("seed", range(N_STREAMED))
def test_random_streamed_sum(gpu, seed):
    """Seeded random rank-ordered sums over 128 - 200 MiB of sources (the
    granule form, from W = 4 with the last lane's cached loads of aligned
    sources aimed at alternating line places): random W, element type, count
    and element offsets, sources all aligned in a third of the cases; every
    element against the oracle."""
    rng = np.random.default_rng([4545, seed])
    W = int(rng.choice([2, 3, 4, 5, 6, 8, 12]))
    dtype = str(rng.choice(["bf16", "f16", "f32"]))
    es = wl.REDUCE_ESIZE[dtype]
    n = int(rng.integers((128 << 20) + 4096, 200 << 20)) // (W * es) + int(rng.integers(0, 700))
    if rng.random() < 0.34:
        in_offs = [int(rng.choice([0, 16, 32, 64, 128])) // es for _ in range(W)]   # 16-byte aligned sources
        out_off = 0
    else:
        in_offs = [int(rng.integers(0, 8)) for _ in range(W)]
        out_off = int(rng.integers(0, 8))
    kind = "bits" if dtype == "f16" or rng.random() < 0.25 else "uniform"
    payloads = wl.reduce_payloads(wl.case_seed(24, seed), W, n, dtype, kind)
    placed = gc.PlacedReduce(payloads, in_offs, out_off, dtype, gpu)
    plan = rog.rog_reduce_plan(placed.srcs, placed.out)
    assert plan["path"] == "multi_wg" and plan["nt_loads"] and plan["shifted_loads"]
    gc.run_reduce_all_paths(placed, "random streamed sum #%d W=%d n=%d %s in=%s out=%d"
                            % (seed, W, n, dtype, in_offs, out_off), paths=(rog.ROG_PATH_AUTO,))
