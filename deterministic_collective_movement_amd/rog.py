"""ctypes binding of librog.so (include/rog.h): argument marshalling only.

Every byte is moved by the library's HIP kernels; this module turns torch
tensors into device pointers, byte counts and the current HIP stream, and
status codes into exceptions.  PyTorch provides device memory and streams.

Entry points keep the C names.  Tensor forms:

* ``rog_gather(srcs, out=None, stream=None)`` -> ``out`` (the same object);
* ``rog_gather_ex(srcs, out, path, stream=None)`` -> ``out``;
* ``rog_gather_many(batch, outs=None, stream=None)`` -> list of outputs;
* ``rog_plan(srcs, out, path=ROG_PATH_AUTO)`` -> dict (no GPU work);
* ``rog_reduce(srcs, out=None, stream=None)`` -> ``out``: the rank-ordered sum
  of W float32, bfloat16 or float16 tensors;
* ``rog_reduce_ex(srcs, out, path, stream=None)``, ``rog_reduce_plan(srcs, out, path)``;
* ``rog_reduce_many(batch, outs=None, stream=None)`` -> list of outputs (one
  launch);
* ``rog_reduce_scatter(inputs, rank, out=None, stream=None)`` -> ``out``: rank
  ``rank``'s share of a reduce-scatter, i.e. ``rog_reduce`` over shard
  ``rank`` of each input (views; nothing is copied).

Raw-pointer forms (``*_ptrs``) take integer device addresses, for callers that
manage their own memory.

Semantics follow RL-Align/RL-Kernel PR #491 ("perf(cuda): vectorize the
deterministic all-gather copy and right-size its single-block path"):
``all_gather(input, out=)`` returns ``out`` itself and hands offset views to
the kernel without copying them (author's replies to the size-test review).
The sum is the reduction of the same PR's deterministic all_reduce /
reduce_scatter ("Not in this PR"); its order and precision are stated in
include/rog.h.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch  # loads the process's HIP runtime before librog.so binds to it

from .build import LIB_PATH

ROG_OK = 0
ROG_ERR_INVALID_ARGUMENT = 1
ROG_ERR_OVERLAP = 2
ROG_ERR_TOO_LARGE = 3
ROG_ERR_LAUNCH = 4

ROG_PATH_AUTO = 0
ROG_PATH_SINGLE_WG = 1
ROG_PATH_MULTI_WG = 2

ROG_PLAN_NT_LOADS = 1
ROG_PLAN_SHIFTED_LOADS = 2

ROG_KERNEL_NONE = 0
ROG_KERNEL_FLAT = 1
ROG_KERNEL_PEER = 2
ROG_KERNEL_REDUCE = 3

ROG_DTYPE_F32 = 0
ROG_DTYPE_BF16 = 1
ROG_DTYPE_F16 = 2

PATH_NAMES = {ROG_PATH_AUTO: "auto", ROG_PATH_SINGLE_WG: "single_wg", ROG_PATH_MULTI_WG: "multi_wg"}
KERNEL_NAMES = {ROG_KERNEL_NONE: "none", ROG_KERNEL_FLAT: "flat", ROG_KERNEL_PEER: "peer",
                ROG_KERNEL_REDUCE: "reduce"}
DTYPES = {torch.float32: ROG_DTYPE_F32, torch.bfloat16: ROG_DTYPE_BF16, torch.float16: ROG_DTYPE_F16}


class RogError(RuntimeError):
    """A non-zero rog_status."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class RogArgumentError(RogError, ValueError):
    pass


class rog_gather_desc(ctypes.Structure):
    _fields_ = [("srcs", ctypes.POINTER(ctypes.c_void_p)),
                ("out", ctypes.c_void_p),
                ("bytes_per_rank", ctypes.c_size_t)]


class rog_reduce_desc(ctypes.Structure):
    _fields_ = [("srcs", ctypes.POINTER(ctypes.c_void_p)),
                ("out", ctypes.c_void_p),
                ("count", ctypes.c_size_t)]


class rog_plan_info(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("grid", ctypes.c_uint32), ("block", ctypes.c_uint32),
                ("vec_ok_mask", ctypes.c_uint64), ("units", ctypes.c_uint64),
                ("peer_magic", ctypes.c_uint32), ("peer_sh1", ctypes.c_uint32),
                ("peer_sh2", ctypes.c_uint32), ("flags", ctypes.c_uint32)]


def _hip_runtimes_mapped() -> set:
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6 and os.path.basename(parts[-1]).startswith("libamdhip64.so"):
                paths.add(os.path.realpath(parts[-1]))
    return paths


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "librog.so is not built (%s); run __graft_entry__.build() or "
            "python -m deterministic_collective_movement_amd.build" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are mapped (%s); librog.so must share torch's"
                          % ", ".join(sorted(runtimes)))
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    ptrs = ctypes.POINTER(ctypes.c_void_p)
    lib.rog_gather.argtypes = [ptrs, i32, sz, vp, vp]
    lib.rog_gather_ex.argtypes = [ptrs, i32, sz, vp, vp, i32]
    lib.rog_gather_many.argtypes = [ctypes.POINTER(rog_gather_desc), i32, i32, vp]
    lib.rog_plan.argtypes = [ptrs, i32, sz, vp, i32, ctypes.POINTER(rog_plan_info)]
    lib.rog_reduce.argtypes = [ptrs, i32, sz, i32, vp, vp]
    lib.rog_reduce_ex.argtypes = [ptrs, i32, sz, i32, vp, vp, i32]
    lib.rog_reduce_plan.argtypes = [ptrs, i32, sz, i32, vp, i32, ctypes.POINTER(rog_plan_info)]
    lib.rog_reduce_many.argtypes = [ctypes.POINTER(rog_reduce_desc), i32, i32, i32, vp]
    for name in ("rog_gather", "rog_gather_ex", "rog_gather_many", "rog_plan", "rog_reduce", "rog_reduce_ex",
                 "rog_reduce_plan", "rog_reduce_many"):
        getattr(lib, name).restype = i32
    for name in ("rog_single_wg_max_bytes", "rog_reduce_single_wg_max_bytes"):
        getattr(lib, name).argtypes = []
        getattr(lib, name).restype = sz
    for name in ("rog_max_peers", "rog_max_batch", "rog_max_batch_pointers", "rog_last_hip_error"):
        getattr(lib, name).argtypes = []
        getattr(lib, name).restype = i32
    lib.rog_status_string.argtypes = [i32]
    lib.rog_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load()


def library_path() -> str:
    return LIB_PATH


def lib() -> ctypes.CDLL:
    return _lib


def _check(status: int, what: str) -> None:
    if status == ROG_OK:
        return
    name = _lib.rog_status_string(status).decode()
    if status == ROG_ERR_LAUNCH:
        raise RogError(status, "%s: %s (hipError_t %d)" % (what, name, _lib.rog_last_hip_error()))
    if status in (ROG_ERR_INVALID_ARGUMENT, ROG_ERR_OVERLAP, ROG_ERR_TOO_LARGE):
        raise RogArgumentError(status, "%s: %s" % (what, name))
    raise RogError(status, "%s: %s" % (what, name))


# ---------------------------------------------------------------------------
# Constants
# ---------------------------------------------------------------------------

def rog_single_wg_max_bytes() -> int:
    return int(_lib.rog_single_wg_max_bytes())


def rog_reduce_single_wg_max_bytes() -> int:
    return int(_lib.rog_reduce_single_wg_max_bytes())


def rog_max_peers() -> int:
    return int(_lib.rog_max_peers())


def rog_max_batch() -> int:
    return int(_lib.rog_max_batch())


def rog_max_batch_pointers() -> int:
    return int(_lib.rog_max_batch_pointers())


def rog_last_hip_error() -> int:
    return int(_lib.rog_last_hip_error())


def rog_status_string(status: int) -> str:
    return _lib.rog_status_string(status).decode()


# ---------------------------------------------------------------------------
# Raw-pointer forms
# ---------------------------------------------------------------------------

def _ptr_array(addrs: Sequence[int]):
    return (ctypes.c_void_p * max(1, len(addrs)))(*addrs)


def rog_gather_ptrs(src_ptrs: Sequence[int], bytes_per_rank: int, out_ptr: int,
                    stream: int = 0, path: int = ROG_PATH_AUTO) -> None:
    """rog_gather_ex on raw device addresses; raises on a non-zero status."""
    st = _lib.rog_gather_ex(_ptr_array(src_ptrs), len(src_ptrs), bytes_per_rank,
                            ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream), path)
    _check(st, "rog_gather")


def rog_plan_ptrs(src_ptrs: Sequence[int], bytes_per_rank: int, out_ptr: int,
                  path: int = ROG_PATH_AUTO) -> dict:
    """rog_plan on raw addresses (no HIP call); raises on a non-zero status."""
    info = rog_plan_info()
    st = _lib.rog_plan(_ptr_array(src_ptrs), len(src_ptrs), bytes_per_rank,
                       ctypes.c_void_p(out_ptr), path, ctypes.byref(info))
    _check(st, "rog_plan")
    return _plan_dict(info)


def rog_status_of_ptrs(src_ptrs: Optional[Sequence[int]], W: int, bytes_per_rank: int,
                       out_ptr: int, path: int = ROG_PATH_AUTO) -> int:
    """Status rog_plan returns for these arguments (``src_ptrs=None`` passes NULL)."""
    info = rog_plan_info()
    arr = None if src_ptrs is None else _ptr_array(src_ptrs)
    return int(_lib.rog_plan(arr, W, bytes_per_rank, ctypes.c_void_p(out_ptr), path,
                             ctypes.byref(info)))


def _plan_dict(info) -> dict:
    return {"path": PATH_NAMES[info.path], "kernel": KERNEL_NAMES[info.kernel],
            "grid": info.grid, "block": info.block, "vec_ok_mask": info.vec_ok_mask,
            "units": info.units, "peer_magic": info.peer_magic, "peer_sh1": info.peer_sh1,
            "peer_sh2": info.peer_sh2, "nt_loads": bool(info.flags & ROG_PLAN_NT_LOADS),
            "shifted_loads": bool(info.flags & ROG_PLAN_SHIFTED_LOADS)}


def rog_reduce_ptrs(src_ptrs: Sequence[int], count: int, dtype: int, out_ptr: int,
                    stream: int = 0, path: int = ROG_PATH_AUTO) -> None:
    """rog_reduce_ex on raw device addresses; raises on a non-zero status."""
    st = _lib.rog_reduce_ex(_ptr_array(src_ptrs), len(src_ptrs), count, dtype,
                            ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream), path)
    _check(st, "rog_reduce")


def rog_reduce_plan_ptrs(src_ptrs: Optional[Sequence[int]], count: int, dtype: int, out_ptr: int,
                         path: int = ROG_PATH_AUTO, W: Optional[int] = None) -> dict:
    """rog_reduce_plan on raw addresses (no HIP call); raises on a non-zero status.
    ``src_ptrs=None`` passes NULL with the given W."""
    info = rog_plan_info()
    arr = None if src_ptrs is None else _ptr_array(src_ptrs)
    st = _lib.rog_reduce_plan(arr, len(src_ptrs) if W is None else W, count, dtype,
                              ctypes.c_void_p(out_ptr), path, ctypes.byref(info))
    _check(st, "rog_reduce_plan")
    return _plan_dict(info)


def rog_reduce_many_ptrs(batch_ptrs: Sequence[Sequence[int]], counts: Sequence[int],
                         out_ptrs: Sequence[int], W: int, dtype: int, stream: int = 0) -> None:
    """rog_reduce_many on raw addresses: tensor t sums the W sources batch_ptrs[t]."""
    n = len(out_ptrs)
    keep = [_ptr_array(p) for p in batch_ptrs]
    descs = (rog_reduce_desc * max(1, n))()
    for t in range(n):
        descs[t].srcs = ctypes.cast(keep[t], ctypes.POINTER(ctypes.c_void_p))
        descs[t].out = ctypes.c_void_p(out_ptrs[t])
        descs[t].count = counts[t]
    st = _lib.rog_reduce_many(descs, n, W, dtype, ctypes.c_void_p(stream))
    _check(st, "rog_reduce_many")


def rog_gather_many_ptrs(batch_ptrs: Sequence[Sequence[int]], sizes: Sequence[int],
                         out_ptrs: Sequence[int], W: int, stream: int = 0) -> None:
    """rog_gather_many on raw addresses: tensor t has W sources batch_ptrs[t]."""
    n = len(out_ptrs)
    keep = [_ptr_array(p) for p in batch_ptrs]
    descs = (rog_gather_desc * max(1, n))()
    for t in range(n):
        descs[t].srcs = ctypes.cast(keep[t], ctypes.POINTER(ctypes.c_void_p))
        descs[t].out = ctypes.c_void_p(out_ptrs[t])
        descs[t].bytes_per_rank = sizes[t]
    st = _lib.rog_gather_many(descs, n, W, ctypes.c_void_p(stream))
    _check(st, "rog_gather_many")


# ---------------------------------------------------------------------------
# Tensor forms
# ---------------------------------------------------------------------------

def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _check_tensor(t: torch.Tensor, what: str, device: torch.device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % what)
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU (got %s)" % (what, t.device))
    if t.get_device() != device.index:
        raise ValueError("%s is on %s, expected %s" % (what, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)


# torch's current stream of a device as a raw handle, without building a
# Stream object (a few microseconds per call otherwise).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream, device) -> int:
    if stream is None:
        if _raw_stream is not None:
            return int(_raw_stream(device.index if device.index is not None else torch.cuda.current_device()))
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return int(stream.cuda_stream)
    return int(stream)


def _prepare(srcs: Sequence[torch.Tensor], out: Optional[torch.Tensor]):
    if len(srcs) == 0:
        raise ValueError("need at least one source tensor")
    _check_tensor(srcs[0], "srcs[0]", srcs[0].device if isinstance(srcs[0], torch.Tensor) else None)
    device = srcs[0].device
    idx = device.index
    S = _nbytes(srcs[0])
    for i, s in enumerate(srcs):
        # one pass of cheap checks; the full check names the first failure
        if not (isinstance(s, torch.Tensor) and s.is_cuda and s.get_device() == idx and s.is_contiguous()):
            _check_tensor(s, "srcs[%d]" % i, device)
        if s.numel() * s.element_size() != S:
            raise ValueError("every source must hold the same number of bytes")
    if out is None:
        out = torch.empty(len(srcs) * S, dtype=torch.uint8, device=device)
    _check_tensor(out, "out", device)
    if _nbytes(out) != len(srcs) * S:
        raise ValueError("out must hold exactly W*S = %d bytes (has %d)" % (len(srcs) * S, _nbytes(out)))
    return device, S, out


# The calling thread's current device index, without torch's lazy-init checks.
_current_device = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device


class _on_device:
    """Make ``device`` the calling thread's current HIP device for the call (the
    library launches on the current device), restoring the previous one."""

    def __init__(self, device: torch.device):
        self.index = device.index if device.index is not None else _current_device()
        self.prev = None

    def __enter__(self):
        cur = _current_device()
        if cur != self.index:
            self.prev = cur
            torch.cuda.set_device(self.index)

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)


def rog_gather_ex(srcs: Sequence[torch.Tensor], out: Optional[torch.Tensor] = None,
                  path: int = ROG_PATH_AUTO, stream=None) -> torch.Tensor:
    """Rank-ordered gather of equal-size tensors into ``out`` with the path forced."""
    device, S, out = _prepare(srcs, out)
    with _on_device(device):
        rog_gather_ptrs([s.data_ptr() for s in srcs], S, out.data_ptr(),
                        _stream_handle(stream, device), path)
    return out


def rog_gather(srcs: Sequence[torch.Tensor], out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """Rank-ordered gather: out[r*S:(r+1)*S] = bytes of srcs[r].  Returns ``out``."""
    return rog_gather_ex(srcs, out, ROG_PATH_AUTO, stream)


def rog_plan(srcs: Sequence[torch.Tensor], out: torch.Tensor, path: int = ROG_PATH_AUTO) -> dict:
    """The launch rog_gather_ex would make for these tensors (no GPU work)."""
    device, S, out = _prepare(srcs, out)
    return rog_plan_ptrs([s.data_ptr() for s in srcs], S, out.data_ptr(), path)


def rog_gather_many(batch: Sequence[Sequence[torch.Tensor]],
                    outs: Optional[Sequence[Optional[torch.Tensor]]] = None,
                    stream=None) -> List[torch.Tensor]:
    """Gather every tensor list ``batch[t]`` (W tensors each) into ``outs[t]``, one launch."""
    n = len(batch)
    if outs is None:
        outs = [None] * n
    if len(outs) != n:
        raise ValueError("one output per tensor")
    if n == 0:
        return []
    W = len(batch[0])
    if any(len(b) != W for b in batch):
        raise ValueError("every tensor of a batch has the same number of sources")
    device = batch[0][0].device
    ready, sizes = [], []
    for t in range(n):
        _, S, o = _prepare(batch[t], outs[t])
        if batch[t][0].device != device:
            raise ValueError("all tensors of a batch must be on one device")
        ready.append(o)
        sizes.append(S)
    with _on_device(device):
        rog_gather_many_ptrs([[s.data_ptr() for s in b] for b in batch], sizes,
                             [o.data_ptr() for o in ready], W, _stream_handle(stream, device))
    return ready


def _prepare_reduce(srcs: Sequence[torch.Tensor], out: Optional[torch.Tensor]):
    if len(srcs) == 0:
        raise ValueError("need at least one source tensor")
    device = srcs[0].device
    dtype = srcs[0].dtype
    if dtype not in DTYPES:
        raise ValueError("rog_reduce sums float32, bfloat16 or float16 tensors (got %s)" % dtype)
    n = srcs[0].numel()
    idx = device.index
    for i, s in enumerate(srcs):
        if not (isinstance(s, torch.Tensor) and s.is_cuda and s.get_device() == idx and s.is_contiguous()):
            _check_tensor(s, "srcs[%d]" % i, device)
        if s.dtype != dtype or s.numel() != n:
            raise ValueError("every source must have the dtype and element count of srcs[0]")
    if out is None:
        out = torch.empty(n, dtype=dtype, device=device)
    _check_tensor(out, "out", device)
    if out.dtype != dtype or out.numel() != n:
        raise ValueError("out must hold %d elements of %s" % (n, dtype))
    return device, n, DTYPES[dtype], out


def rog_reduce_ex(srcs: Sequence[torch.Tensor], out: Optional[torch.Tensor] = None,
                  path: int = ROG_PATH_AUTO, stream=None) -> torch.Tensor:
    """Rank-ordered sum of equal-shape tensors into ``out`` with the path forced."""
    device, n, dt, out = _prepare_reduce(srcs, out)
    with _on_device(device):
        rog_reduce_ptrs([s.data_ptr() for s in srcs], n, dt, out.data_ptr(),
                        _stream_handle(stream, device), path)
    return out


def rog_reduce(srcs: Sequence[torch.Tensor], out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """out[i] = rank-ordered binary32 sum of srcs[r][i], rounded to the tensors'
    dtype (float32, bfloat16 or float16).  ``out`` may be one of ``srcs`` (in
    place)."""
    return rog_reduce_ex(srcs, out, ROG_PATH_AUTO, stream)


def rog_reduce_plan(srcs: Sequence[torch.Tensor], out: torch.Tensor, path: int = ROG_PATH_AUTO) -> dict:
    """The launch rog_reduce_ex would make for these tensors (no GPU work)."""
    device, n, dt, out = _prepare_reduce(srcs, out)
    return rog_reduce_plan_ptrs([s.data_ptr() for s in srcs], n, dt, out.data_ptr(), path)


def rog_reduce_scatter(inputs: Sequence[torch.Tensor], rank: int, out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Rank ``rank``'s share of a reduce-scatter over the W ``inputs``: each input
    holds W shards of n elements; out = rog_reduce over shard ``rank`` of every
    input (views into the inputs, no copy)."""
    W = len(inputs)
    if W == 0:
        raise ValueError("need at least one input")
    if not 0 <= rank < W:
        raise ValueError("rank must be in [0, %d)" % W)
    total = inputs[0].numel()
    if total % W:
        raise ValueError("each input must hold W equal shards (numel %% W == 0)")
    n = total // W
    for i, t in enumerate(inputs):
        _check_tensor(t, "inputs[%d]" % i, inputs[0].device)
    return rog_reduce([t.reshape(-1)[rank * n:(rank + 1) * n] for t in inputs], out, stream)


def rog_reduce_many(batch: Sequence[Sequence[torch.Tensor]],
                    outs: Optional[Sequence[Optional[torch.Tensor]]] = None,
                    stream=None) -> List[torch.Tensor]:
    """Rank-ordered sums of every tensor list ``batch[t]`` (W tensors each, one
    dtype for the batch) into ``outs[t]``, in one launch."""
    n = len(batch)
    if outs is None:
        outs = [None] * n
    if len(outs) != n:
        raise ValueError("one output per tensor")
    if n == 0:
        return []
    W = len(batch[0])
    if any(len(b) != W for b in batch):
        raise ValueError("every tensor of a batch has the same number of sources")
    device = batch[0][0].device
    ready, counts, dt0 = [], [], None
    for t in range(n):
        dev, count, dt, o = _prepare_reduce(batch[t], outs[t])
        if dev != device:
            raise ValueError("all tensors of a batch must be on one device")
        if dt0 is not None and dt != dt0:
            raise ValueError("all tensors of a batch must have one dtype")
        dt0 = dt
        ready.append(o)
        counts.append(count)
    with _on_device(device):
        rog_reduce_many_ptrs([[s.data_ptr() for s in b] for b in batch], counts,
                             [o.data_ptr() for o in ready], W, dt0, _stream_handle(stream, device))
    return ready
