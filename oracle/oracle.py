"""CPU oracle for the rank-ordered gather and the rank-ordered sum (Python side).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code with
the HIP library (``deterministic_collective_movement_amd``) and never imports it.

Two independent implementations of one definition:

* ``gather_c`` / ``gather_many_c`` call ``rog_oracle.c`` (plain C, built with
  gcc by ``build_oracle``): a per-peer byte loop in rank order.
* ``gather_py`` is a pure-Python per-byte loop for tiny inputs.

The rank-ordered sum (the reduction of a deterministic all-reduce or
reduce-scatter) likewise has a C form, ``reduce_c``, and a pure-Python form,
``reduce_py``, which rounds every binary32 addition through ``struct`` (an
addition of two binary32 numbers in binary64 followed by one rounding to
binary32 is the correctly rounded binary32 sum: 53 >= 2*24 + 2), rounds to
bf16 with its own integer arithmetic and to binary16 through ``struct``'s half
format.  The reading of the pages it follows is
stated in ``rog_oracle.c``: the pages name their reduction a fixed tree but
print neither its order nor its precision, so the sum is PARITY UNPINNED
against the pages' own order; its pins fix the left-deep rank-order chain in
binary32 that this library defines.

Definition (RL-Align/RL-Kernel PR #491, "perf(cuda): vectorize the deterministic
all-gather copy and right-size its single-block path", section "What", the
copy_rank_ordered bullet): the faster copy changes how bytes move, not which
bytes land where, so the result is that of an all-gather: payload r at byte
offset r*S of the output.  The batched form follows the same PR's description of
all_gather_many: every tensor of the list gets its own gathered output.
"""
from __future__ import annotations

import ctypes
import math
import os
import struct
import subprocess
from typing import List, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rog_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build_oracle(force: bool = True) -> str:
    """Compile rog_oracle.c into oracle/liboracle.so with gcc -O2."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
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
        for name, ct in (("rog_oracle_reduce_f32", ctypes.c_void_p), ("rog_oracle_reduce_bf16", ctypes.c_void_p),
                         ("rog_oracle_reduce_f16", ctypes.c_void_p)):
            f = getattr(lib, name)
            f.restype = None
            f.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_size_t, ct]
        for name in ("rog_oracle_f32_to_bf16", "rog_oracle_f32_to_f16"):
            getattr(lib, name).restype = ctypes.c_uint16
            getattr(lib, name).argtypes = [ctypes.c_float]
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


# ---------------------------------------------------------------------------
# Rank-ordered sum
# ---------------------------------------------------------------------------

#: Element types of the sum: numpy storage dtype of one element.
REDUCE_DTYPES = {"f32": np.dtype(np.float32), "bf16": np.dtype(np.uint16), "f16": np.dtype(np.uint16)}


def reduce_c(srcs: Sequence[np.ndarray], out: np.ndarray, dtype: str) -> np.ndarray:
    """out[i] = rank-ordered binary32 sum of srcs[r][i], rounded to ``dtype``.

    ``dtype`` "f32": float32 arrays; "bf16" / "f16": uint16 arrays holding
    bf16 / IEEE binary16 bits.
    All arrays 1-D, equal length, aligned to their element size.
    """
    want = REDUCE_DTYPES[dtype]
    W = len(srcs)
    if W < 1:
        raise ValueError("need at least one payload")
    n = out.shape[0]
    for a in list(srcs) + [out]:
        if a.dtype != want or a.ndim != 1 or a.shape[0] != n:
            raise ValueError("reduce_c wants 1-D %s arrays of one length" % want)
        if a.ctypes.data % want.itemsize:
            raise ValueError("elements must be aligned to their size")
    if not out.flags.writeable:
        raise ValueError("out must be writeable")
    ptrs = (ctypes.c_void_p * W)(*[a.ctypes.data for a in srcs])
    fn = {"f32": _load().rog_oracle_reduce_f32, "bf16": _load().rog_oracle_reduce_bf16,
          "f16": _load().rog_oracle_reduce_f16}[dtype]
    fn(ptrs, W, n, out.ctypes.data)
    return out


def f32_to_bf16_c(x: np.ndarray) -> np.ndarray:
    """The C oracle's binary32 -> bf16 rounding, element by element (uint16 bits)."""
    lib = _load()
    return np.array([lib.rog_oracle_f32_to_bf16(float(v)) for v in np.asarray(x, np.float32)], np.uint16)


#: Magnitudes from which rounding to binary32 gives infinity: the midpoint
#: between the largest binary32 number, (2 - 2^-23) 2^127, and 2^128; that
#: largest number has an odd significand, so the tie itself rounds up.
_F32_OVERFLOW = 2.0 ** 128 - 2.0 ** 103


def f32_to_f16_c(x: np.ndarray) -> np.ndarray:
    """The C oracle's binary32 -> binary16 rounding, element by element (uint16 bits)."""
    lib = _load()
    return np.array([lib.rog_oracle_f32_to_f16(float(v)) for v in np.asarray(x, np.float32)], np.uint16)


#: Magnitudes from which rounding to binary16 gives infinity: the midpoint
#: between the largest binary16 number, 65504 (odd significand), and 2^16.
_F16_OVERFLOW = 65520.0


def f16_bits_to_float(h: int) -> float:
    return struct.unpack("<e", struct.pack("<H", h & 0xFFFF))[0]


def f32_to_f16_py(x: float) -> int:
    """binary32 value -> binary16 bits, nearest-even (struct's half format
    rounds half to even; overflow to infinity handled here); a NaN becomes a
    quiet NaN with the same sign."""
    if math.isnan(x):
        return 0xFE00 if math.copysign(1.0, x) < 0 else 0x7E00
    if abs(x) >= _F16_OVERFLOW:
        return 0xFC00 if x < 0 else 0x7C00
    return struct.unpack("<H", struct.pack("<e", x))[0]


def _f32(x: float) -> float:
    """Round a Python float (binary64) to the nearest binary32, ties to even."""
    if not math.isnan(x) and abs(x) >= _F32_OVERFLOW:
        return math.copysign(math.inf, x)
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bf16_bits_to_float(h: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (h & 0xFFFF) << 16))[0]


def f32_to_bf16_py(x: float) -> int:
    """binary32 value -> bf16 bits, nearest-even on the dropped 16 bits; a NaN
    becomes a quiet NaN with the same sign (payload not specified)."""
    u = _f32_bits(x)
    if math.isnan(x):
        return ((u >> 16) | 0x0040) & 0xFFFF
    upper, dropped = u >> 16, u & 0xFFFF
    if dropped > 0x8000 or (dropped == 0x8000 and upper & 1):
        upper += 1
    return upper & 0xFFFF


def reduce_py(srcs: Sequence[Sequence], dtype: str) -> List:
    """Pure-Python rank-ordered sum, element by element (tiny inputs only).

    "f32": sequences of Python floats that are binary32 values; returns floats.
    "bf16" / "f16": sequences of bf16 / binary16 bit patterns (ints); returns
    bit patterns of the same type.
    """
    widen = {"bf16": bf16_bits_to_float, "f16": f16_bits_to_float}.get(dtype)
    narrow = {"bf16": f32_to_bf16_py, "f16": f32_to_f16_py}.get(dtype)
    W = len(srcs)
    n = len(srcs[0])
    out = []
    for i in range(n):
        if dtype == "f32":
            acc = _f32(float(srcs[0][i]))
            for r in range(1, W):
                acc = _f32(acc + _f32(float(srcs[r][i])))
            out.append(acc)
        else:
            acc = widen(int(srcs[0][i]))
            for r in range(1, W):
                acc = _f32(acc + widen(int(srcs[r][i])))
            out.append(narrow(acc))
    return out
