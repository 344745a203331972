"""Helpers of the GPU parity tests: place a case's payloads in guarded device
buffers, run the library through its C ABI, and compare every byte of every
guarded buffer with the CPU oracle's result (gathers), or every element of the
output with the oracle's rank-ordered sum, bit for bit (sums)."""
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


def _sync(t: torch.Tensor) -> None:
    """Wait for the GPU work on t's device; nothing to wait for on the CPU,
    where the harness's own mutation tests run it."""
    if t.device.type == "cuda":
        torch.cuda.synchronize(t.device)


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
            d = torch.from_numpy(h).to(device, copy=True)   # never an alias of h, also on the CPU
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
        _sync(self.out_dev)
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


# ---------------------------------------------------------------------------
# Rank-ordered sum
# ---------------------------------------------------------------------------

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _same_elements(got: np.ndarray, want: np.ndarray, dtype: str) -> np.ndarray:
    """Per element: equal bits, or both NaN (NaN payloads are not specified)."""
    if dtype == "f32":
        g, w = got.view(np.uint32), want.view(np.uint32)
        gn = (g & 0x7FFFFFFF) > 0x7F800000
        wn = (w & 0x7FFFFFFF) > 0x7F800000
    else:
        inf = 0x7F80 if dtype == "bf16" else 0x7C00
        g, w = got.view(np.uint16), want.view(np.uint16)
        gn = (g & 0x7FFF) > inf
        wn = (w & 0x7FFF) > inf
    return (g == w) | (gn & wn)


class PlacedReduce:
    """A rank-ordered sum's payloads and output in guarded byte buffers, each at
    an element offset, on host and device."""

    def __init__(self, payloads: Sequence[np.ndarray], in_offs: Sequence[int], out_off: int,
                 dtype: str, device: torch.device, in_place: int = -1):
        self.W = len(payloads)
        self.n = int(payloads[0].shape[0])
        self.dtype = dtype
        self.es = wl.REDUCE_ESIZE[dtype]
        self.payloads = [np.ascontiguousarray(p) for p in payloads]
        self.out_off = out_off
        self.in_place = in_place
        nb = self.n * self.es
        self.src_host, self.src_dev, self.srcs = [], [], []
        for p, o in zip(self.payloads, in_offs):
            h = guarded_host(nb, o * self.es)
            start = wl.GUARD + o * self.es
            h[start:start + nb] = p.view(np.uint8)
            d = torch.from_numpy(h).to(device, copy=True)   # never an alias of h, also on the CPU
            self.src_host.append(h)
            self.src_dev.append(d)
            self.srcs.append(d[start:start + nb].view(TORCH_DTYPES[dtype]))
        self.out_start = wl.GUARD + out_off * self.es
        self.out_dev = torch.full((self.out_start + nb + wl.GUARD,), wl.GUARD_BYTE, dtype=torch.uint8,
                                  device=device)
        self.out = self.out_dev[self.out_start:self.out_start + nb].view(TORCH_DTYPES[dtype])
        if in_place >= 0:
            # the output is source `in_place` itself
            self.out_dev = self.src_dev[in_place]
            self.out_start = wl.GUARD + in_offs[in_place] * self.es
            self.out = self.srcs[in_place]
        self._expected = None

    def expected(self) -> np.ndarray:
        if self._expected is None:
            want = np.empty(self.n, dtype=oracle.REDUCE_DTYPES[self.dtype])
            oracle.reduce_c(self.payloads, want, self.dtype)
            self._expected = want
        return self._expected

    def reset(self) -> None:
        if self.in_place >= 0:
            h = self.src_host[self.in_place]
            self.out_dev.copy_(torch.from_numpy(h))
        else:
            self.out_dev.fill_(wl.GUARD_BYTE)

    def check(self, label: str) -> None:
        _sync(self.out_dev)
        buf = self.out_dev.cpu().numpy()
        nb = self.n * self.es
        # Outside [out_start, out_start + nb) the buffer must be as it was: the
        # guards, and for an in-place sum the source buffer's own guards.
        before = self.src_host[self.in_place] if self.in_place >= 0 else None
        pre, post = buf[:self.out_start], buf[self.out_start + nb:]
        if before is None:
            intact = np.all(pre == wl.GUARD_BYTE) and np.all(post == wl.GUARD_BYTE)
        else:
            intact = (np.array_equal(pre, before[:self.out_start])
                      and np.array_equal(post, before[self.out_start + nb:]))
        if not intact:
            raise AssertionError("%s: a guard byte changed" % label)
        got = buf[self.out_start:self.out_start + nb].copy().view(oracle.REDUCE_DTYPES[self.dtype])
        ok = _same_elements(got, self.expected(), self.dtype)
        if not ok.all():
            i = int(np.flatnonzero(~ok)[0])
            bits = np.uint32 if self.es == 4 else np.uint16
            raise AssertionError("%s: %d of %d elements differ; first %d: got %s want %s"
                                 % (label, int((~ok).sum()), self.n, i, hex(int(got.view(bits)[i])),
                                    hex(int(self.expected().view(bits)[i]))))
        for r, (h, d) in enumerate(zip(self.src_host, self.src_dev)):
            if r == self.in_place:
                continue
            if not np.array_equal(d.cpu().numpy(), h):
                raise AssertionError("%s: source buffer %d changed" % (label, r))


def place_reduce(case: wl.ReduceCase, device) -> PlacedReduce:
    return PlacedReduce(case.payloads(), case.in_offs, case.out_off, case.dtype, device)


def run_reduce_all_paths(placed: PlacedReduce, label: str, paths=PATHS) -> None:
    for path in paths:
        placed.reset()
        print("%s path=%s" % (label, rog.PATH_NAMES[path]), flush=True)
        ret = rog.rog_reduce_ex(placed.srcs, placed.out, path)
        assert ret is placed.out
        placed.check("%s path=%s" % (label, rog.PATH_NAMES[path]))


class PlacedReduceBatch:
    """A batch of rank-ordered sums: tensor t's W payloads and output, each in
    guarded buffers at element offsets."""

    def __init__(self, items: Sequence[PlacedReduce]):
        self.items = list(items)

    def run(self, label: str) -> None:
        for it in self.items:
            it.reset()
        print(label, flush=True)
        outs = rog.rog_reduce_many([it.srcs for it in self.items], [it.out for it in self.items])
        for o, it in zip(outs, self.items):
            assert o is it.out
        for t, it in enumerate(self.items):
            it.check("%s tensor %d (n=%d, %s)" % (label, t, it.n, it.dtype))

