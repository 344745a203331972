"""CPU oracle for the rank-ordered gather (Python side).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code with
the HIP library (``deterministic_collective_movement_amd``) and never imports it.

Two independent implementations of one definition:

* ``gather_c`` / ``gather_many_c`` call ``rog_oracle.c`` (plain C, built with
  gcc by ``build_oracle``): a per-peer byte loop in rank order.
* ``gather_py`` is a pure-Python per-byte loop for tiny inputs.

Definition (RL-Align/RL-Kernel PR #491, "perf(cuda): vectorize the deterministic
all-gather copy and right-size its single-block path", section "What", the
copy_rank_ordered bullet): the copy is a pure rank-ordered copy with a
byte-identical result, i.e. an all-gather whose output holds payload r at byte
offset r*S.  The batched form follows the same PR's description of
all_gather_many: every tensor of the list gets its own gathered output.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rog_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build_oracle(force: bool = True) -> str:
    """Compile rog_oracle.c into oracle/liboracle.so with gcc -O2."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-Werror", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_oracle(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.rog_oracle_gather.restype = None
        lib.rog_oracle_gather.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                          ctypes.c_size_t, ctypes.c_void_p]
        lib.rog_oracle_gather_many.restype = None
        lib.rog_oracle_gather_many.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                               ctypes.POINTER(ctypes.c_void_p),
                                               ctypes.POINTER(ctypes.c_size_t),
                                               ctypes.c_int, ctypes.c_int]
        _lib = lib
    return _lib


def _addr(a: np.ndarray) -> int:
    if a.dtype != np.uint8 or a.ndim != 1:
        raise TypeError("oracle buffers are 1-D uint8 arrays")
    return a.ctypes.data


def gather_c(srcs: Sequence[np.ndarray], out: np.ndarray) -> np.ndarray:
    """Rank-ordered gather of W equal-length uint8 payloads into ``out`` (W*S bytes).

    ``srcs`` and ``out`` may be views at any byte offset of larger arrays.
    """
    W = len(srcs)
    if W < 1:
        raise ValueError("need at least one payload")
    S = srcs[0].shape[0]
    if any(s.shape[0] != S for s in srcs):
        raise ValueError("payloads must all hold S bytes")
    if out.shape[0] != W * S:
        raise ValueError("out must hold exactly W*S bytes")
    if not out.flags.writeable:
        raise ValueError("out must be writeable")
    ptrs = (ctypes.c_void_p * W)(*[_addr(s) for s in srcs])
    _load().rog_oracle_gather(ptrs, W, S, _addr(out))
    return out


def gather_many_c(batch: Sequence[Sequence[np.ndarray]], outs: Sequence[np.ndarray]) -> list:
    """Batched gather: tensor t's payloads ``batch[t]`` (W each) into ``outs[t]``."""
    n = len(batch)
    if n != len(outs):
        raise ValueError("one output per tensor")
    if n == 0:
        return list(outs)
    W = len(batch[0])
    if any(len(b) != W for b in batch):
        raise ValueError("all tensors of a batch share W")
    sizes = []
    flat = []
    for srcs, out in zip(batch, outs):
        S = srcs[0].shape[0]
        if any(s.shape[0] != S for s in srcs) or out.shape[0] != W * S:
            raise ValueError("payload/output size mismatch")
        sizes.append(S)
        flat.extend(_addr(s) for s in srcs)
    p = (ctypes.c_void_p * len(flat))(*flat)
    o = (ctypes.c_void_p * n)(*[_addr(x) for x in outs])
    sz = (ctypes.c_size_t * n)(*sizes)
    _load().rog_oracle_gather_many(p, o, sz, n, W)
    return list(outs)


def gather_py(srcs: Sequence[bytes], S: int) -> bytearray:
    """Pure-Python per-byte rank-ordered gather; for tiny inputs only."""
    W = len(srcs)
    out = bytearray(W * S)
    for r in range(W):
        src = srcs[r]
        for i in range(S):
            out[r * S + i] = src[i]
    return out
