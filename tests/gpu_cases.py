"""Helpers of the GPU parity tests: place a case's payloads in guarded device
buffers, run the library through its C ABI, and compare every byte of every
guarded buffer with the CPU oracle's result."""
from __future__ import annotations

from typing import List, Sequence

import numpy as np
import torch

from deterministic_collective_movement_amd import rog
from deterministic_collective_movement_amd import workloads as wl
from oracle import oracle

PATHS = (rog.ROG_PATH_AUTO, rog.ROG_PATH_SINGLE_WG, rog.ROG_PATH_MULTI_WG)


def guarded_host(nbytes: int, off: int) -> np.ndarray:
    return np.full(wl.GUARD + off + nbytes + wl.GUARD, wl.GUARD_BYTE, dtype=np.uint8)


class Placed:
    """A gather's payloads and output in guarded buffers, on host and device."""

    def __init__(self, payloads: Sequence[np.ndarray], in_offs: Sequence[int], out_off: int,
                 device: torch.device):
        self.W = len(payloads)
        self.S = int(payloads[0].shape[0])
        self.payloads = list(payloads)
        self.in_offs = list(in_offs)
        self.out_off = out_off
        self.src_host, self.src_dev, self.srcs = [], [], []
        for p, o in zip(payloads, in_offs):
            h = guarded_host(self.S, o)
            h[wl.GUARD + o: wl.GUARD + o + self.S] = p
            d = torch.from_numpy(h).to(device)
            self.src_host.append(h)
            self.src_dev.append(d)
            self.srcs.append(d[wl.GUARD + o: wl.GUARD + o + self.S])
        self.out_dev = torch.full((wl.GUARD + out_off + self.W * self.S + wl.GUARD,),
                                  wl.GUARD_BYTE, dtype=torch.uint8, device=device)
        self.out = self.out_dev[wl.GUARD + out_off: wl.GUARD + out_off + self.W * self.S]
        self._expected = None

    def expected(self) -> np.ndarray:
        """The whole guarded output buffer as the oracle computes it."""
        if self._expected is None:
            e = guarded_host(self.W * self.S, self.out_off)
            start = wl.GUARD + self.out_off
            oracle.gather_c(self.payloads, e[start:start + self.W * self.S])
            self._expected = e
        return self._expected

    def reset_output(self) -> None:
        self.out_dev.fill_(wl.GUARD_BYTE)

    def check(self, label: str) -> None:
        torch.cuda.synchronize()
        got = self.out_dev.cpu().numpy()
        want = self.expected()
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got != want)
            start = wl.GUARD + self.out_off
            first = int(bad[0])
            where = ("prefix guard" if first < start else
                     "suffix guard" if first >= start + self.W * self.S else
                     "output byte %d (rank %d, index %d)" % (first - start, (first - start) // max(1, self.S),
                                                             (first - start) % max(1, self.S)))
            raise AssertionError("%s: %d bytes differ; first at %s: got %d want %d"
                                 % (label, bad.size, where, got[first], want[first]))
        for r, (h, d) in enumerate(zip(self.src_host, self.src_dev)):
            if not np.array_equal(d.cpu().numpy(), h):
                raise AssertionError("%s: source buffer %d changed" % (label, r))


def place_case(case: wl.GatherCase, device) -> Placed:
    return Placed([case.payload(r) for r in range(case.W)], case.in_offs, case.out_off, device)


def run_all_paths(placed: Placed, label: str, paths=PATHS) -> None:
    for path in paths:
        placed.reset_output()
        print("%s path=%s" % (label, rog.PATH_NAMES[path]), flush=True)
        ret = rog.rog_gather_ex(placed.srcs, placed.out, path)
        assert ret is placed.out
        placed.check("%s path=%s" % (label, rog.PATH_NAMES[path]))


class PlacedBatch:
    """A batch: tensor t's W payloads and output, each in guarded buffers."""

    def __init__(self, W: int, payloads: List[List[np.ndarray]], in_offs: Sequence[int],
                 out_offs: Sequence[int], device):
        self.items = [Placed(p, [io] * W, oo, device) for p, io, oo in zip(payloads, in_offs, out_offs)]
        self.W = W

    def run(self, label: str) -> None:
        for it in self.items:
            it.reset_output()
        print(label, flush=True)
        outs = rog.rog_gather_many([it.srcs for it in self.items], [it.out for it in self.items])
        for o, it in zip(outs, self.items):
            assert o is it.out
        for t, it in enumerate(self.items):
            it.check("%s tensor %d (S=%d, in=%d, out=%d)" % (label, t, it.S, it.in_offs[0], it.out_off))


def place_batch(case: wl.BatchCase, device) -> PlacedBatch:
    payloads = [[case.payload(t, r) for r in range(case.W)] for t in range(len(case.tensors))]
    return PlacedBatch(case.W, payloads, [x.in_off for x in case.tensors],
                       [x.out_off for x in case.tensors], device)
