#!/usr/bin/env python3
"""Benchmark of the rank-ordered gather on one MI355X.

One step is one rog_gather of the bandwidth workload: W = 8 payloads of
64 MiB (bf16 values uniform in [-1, 1]) gathered into a 512 MiB output, with
inputs and output resident in HBM before the timed region.  The bytes one step
moves are 2*W*S (every payload byte read once, every output byte written once).

The timed region is K back-to-back calls bracketed by device synchronisation and
two HIP events on the calls' stream (torch.cuda.Event on torch's current stream,
which the calls use); ``value`` and the kernel's average launch duration come
from it.  A second, untimed pass brackets every call with its own events, as
the pages time each call (RL-Align/RL-Kernel PR #491, "Results": median of 100
calls), for the per-call p50.

Besides the headline line the run measures: the same gather with every payload
and the output at odd byte offsets (the per-payload path); small gathers (the
pages' 1 - 128 KiB per-rank sizes at 2 and 8 payloads), per call, replayed
from a HIP graph of 100 calls, and timed from C by bench_native.c (a child
process), next to the eager floor of one tiny torch kernel timed the same way;
the batched gather (16 tensors, W = 4, one launch, after 40 untimed calls); the device-to-device copy
ceiling and the HBM figure the HIP runtime reports; aligned gathers with
2 - 512 MiB outputs, warm and with rotating buffer sets (cold), beside the
bound one launch per gather allows (from bench_floor, a child process); the
rank-ordered sum (rog_reduce: W = 8 bf16 payloads of 64 MiB, aligned and one
element off, the pages' per-rank sizes of 1 KiB - 4 MiB at W = 2 and 8, a
16-tensor rog_reduce_many, and W = 8 and 3 with the sources placed three ways
in memory); the headline gather and the W = 8 sum in four
cache states (back to back on one set, over four rotating sets, and after a
1 GiB read-only or read-write pass over other memory); and the CPU oracle on bounded samples of the
headline gather and of the large sum (the CPU-baseline legs, the only ones
that call the oracle).

Prints ONE JSON line.  ``--gpus N`` with N > 1 exits: the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "rank-ordered gather HBM GB/s (% of peak) + p50 µs at 1–128 KiB/payload"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, AMD's published peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "flat_kernel_w8x64MiB_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "deterministic_collective_movement_amd", "csrc", f)
                  for f in ("rog_kernels.hip", "rog_internal.h", "rog_plan.cpp", "rog_device.h")]
LATENCY_SIZES_KIB = (1, 8, 32, 128)
# Calls timed per small-payload latency case, whatever --steps is: the pages
# report the median of 100 calls (RL-Align/RL-Kernel PR #491, "Results").
LATENCY_CALLS = 100
LATENCY_WARMUP = 10
NATIVE_SRC = os.path.join(ROOT, "bench_native.c")
NATIVE_BIN = os.path.join(ROOT, "_build", "bench_native")
FLOOR_SRC = os.path.join(ROOT, "bench_floor.hip")
FLOOR_BIN = os.path.join(ROOT, "_build", "bench_floor")


def build_native() -> str:
    """Compile bench_native.c (the small-gather latency timed from C) against
    librog.so and the HIP runtime into _build/bench_native."""
    import subprocess
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    pkg = os.path.join(ROOT, "deterministic_collective_movement_amd")
    os.makedirs(os.path.dirname(NATIVE_BIN), exist_ok=True)
    tmp = NATIVE_BIN + ".tmp%d" % os.getpid()
    subprocess.check_call([
        "gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), NATIVE_SRC,
        os.path.join(pkg, "librog.so"), "-Wl,-rpath,$ORIGIN/../deterministic_collective_movement_amd",
        "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", tmp])
    os.replace(tmp, NATIVE_BIN)
    # the launch-floor harness (null, load-only and store-only kernels of the
    # gathers' launch shape), for the profiles; bench.py does not run it
    hipcc = os.path.join(rocm, "bin", "hipcc")
    tmp = FLOOR_BIN + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc, "-O3", "-std=c++17", "-Wall", "-Wextra", "-Werror", "--offload-arch=gfx950",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "-Wno-unused-command-line-argument", FLOOR_SRC, "-o", tmp],
                          stderr=subprocess.DEVNULL)
    os.replace(tmp, FLOOR_BIN)
    return NATIVE_BIN


def latency_native(timeout_s=120):
    """Run the native latency harness in a child process; its JSON, or why not."""
    import subprocess
    if not os.path.exists(NATIVE_BIN):
        return {"error": "bench_native not built"}
    try:
        r = subprocess.run([NATIVE_BIN], capture_output=True, text=True, timeout=timeout_s)
    except subprocess.TimeoutExpired:
        return {"error": "timed out"}
    if r.returncode != 0:
        return {"error": "exit %d: %s" % (r.returncode, r.stderr.strip()[-200:])}
    return json.loads(r.stdout)


def launch_floor_native(timeout_s=60):
    """Run the launch-floor harness (``bench_floor``, built beside
    ``bench_native``) in a child process: per kernel (null, load, store) and
    grid, the µs per launch eagerly and replayed back to back from a graph."""
    import subprocess
    if not os.path.exists(FLOOR_BIN):
        return {"error": "bench_floor not built"}
    try:
        r = subprocess.run([FLOOR_BIN], capture_output=True, text=True, timeout=timeout_s)
    except subprocess.TimeoutExpired:
        return {"error": "timed out"}
    if r.returncode != 0:
        return {"error": "exit %d: %s" % (r.returncode, r.stderr.strip()[-200:])}
    return [json.loads(line) for line in r.stdout.splitlines() if line.strip()]


# ---------------------------------------------------------------------------
# Pure helpers (CPU-testable)
# ---------------------------------------------------------------------------

def one_launch_bound(rows, floor_us, lo_mib=128, hi_mib=512):
    """The best a cold gather of each ``bandwidth_sweep`` row could do with one
    launch per gather: its bytes at the cold streaming rate the same sweep
    measures between ``lo_mib`` and ``hi_mib`` of output (difference of the
    times per gather, per W), plus ``floor_us``, the cost of an empty launch
    back to back.  Per W: the rate, and per row the bound in µs and in % of
    the peak beside the measured cold figure."""
    by_w = {}
    for r in rows:
        by_w.setdefault(r["W"], {})[r["out_MiB"]] = r
    out = {"floor_us_per_launch": round(floor_us, 3), "cold_stream_GBps": {}, "rows": []}
    for W, rs in sorted(by_w.items()):
        if lo_mib not in rs or hi_mib not in rs:
            continue
        lo, hi = rs[lo_mib], rs[hi_mib]
        dt_us = hi["cold_us_per_gather"] - lo["cold_us_per_gather"]
        if dt_us <= 0:
            continue
        rate = 2 * (hi_mib - lo_mib) * (1 << 20) / (dt_us * 1e3)          # GB/s
        out["cold_stream_GBps"][str(W)] = round(rate, 1)
        for mib in sorted(rs):
            moved = 2 * mib * (1 << 20)
            bound_us = moved / (rate * 1e3) + floor_us
            out["rows"].append({"W": W, "out_MiB": mib, "bound_us": round(bound_us, 2),
                                "bound_pct_of_peak": round(100 * moved / (bound_us * 1e3) / PEAK_HBM_GBPS, 1),
                                "cold_us_per_gather": rs[mib]["cold_us_per_gather"],
                                "cold_pct_of_peak": rs[mib]["cold_pct_of_peak"]})
    return out


def percentile(xs, q):
    """Linear-interpolated percentile (q in [0, 100]) of a non-empty sequence."""
    s = sorted(xs)
    if not s:
        raise ValueError("empty sample")
    k = (len(s) - 1) * q / 100.0
    lo = int(k)
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (k - lo)


def summarize_ms(samples_ms):
    return {"p10_us": 1e3 * percentile(samples_ms, 10), "p50_us": 1e3 * percentile(samples_ms, 50),
            "p90_us": 1e3 * percentile(samples_ms, 90), "mean_us": 1e3 * statistics.fmean(samples_ms),
            "n": len(samples_ms)}


def gbps(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def code_only(text):
    """C/C++ source with comments removed and whitespace runs collapsed, so
    that edits to comments alone leave the digest of the code unchanged.  (The
    sources hold no string literal with a comment marker in it.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest(paths=KERNEL_SOURCES):
    """sha256 over the code (comments and layout stripped) of the sources the
    headline kernel is built from, in order."""
    h = hashlib.sha256()
    for p in paths:
        with open(p) as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()


def read_traffic(path=TRAFFIC_FILE, digest=None):
    """HBM bytes per launch of the headline kernel from the committed counter
    summary, or None when there is none or the kernel sources changed since the
    counters were taken."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_d = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_d or not m_t:
        return None
    if m_d.group(1) != (digest or kernel_source_digest()):
        return None
    return float(m_t.group(1))


def roofline(alg_bytes, mean_launch_ms, traffic):
    achieved = gbps(alg_bytes, mean_launch_ms)
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": None if traffic is None else int(traffic)}


def build_line(*, value, steps, warmup, ms_per_step, config, roof, cpu, extras):
    line = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": config, "roofline": roof, "cpu_baseline": cpu}
    line.update(extras)
    return line


# ---------------------------------------------------------------------------
# GPU measurement
# ---------------------------------------------------------------------------

class Call:
    """A prepared rog_gather call: ctypes arguments built once."""

    def __init__(self, rog, srcs, out, stream):
        self.lib = rog.lib()
        self.W = len(srcs)
        self.S = srcs[0].numel() * srcs[0].element_size()
        self.ptrs = (ctypes.c_void_p * self.W)(*[s.data_ptr() for s in srcs])
        self.out = ctypes.c_void_p(out.data_ptr())
        self.stream = ctypes.c_void_p(stream)

    def __call__(self):
        st = self.lib.rog_gather(self.ptrs, self.W, self.S, self.out, self.stream)
        if st != 0:
            raise RuntimeError("rog_gather failed with status %d" % st)


class BatchCall:
    """A prepared rog_gather_many call: descriptor array built once."""

    def __init__(self, rog, batch, outs, stream):
        self.lib = rog.lib()
        self.W = len(batch[0])
        self.n = len(batch)
        self.keep = [(ctypes.c_void_p * self.W)(*[s.data_ptr() for s in srcs]) for srcs in batch]
        self.descs = (rog.rog_gather_desc * self.n)()
        for t, (srcs, out) in enumerate(zip(batch, outs)):
            self.descs[t].srcs = ctypes.cast(self.keep[t], ctypes.POINTER(ctypes.c_void_p))
            self.descs[t].out = ctypes.c_void_p(out.data_ptr())
            self.descs[t].bytes_per_rank = srcs[0].numel() * srcs[0].element_size()
        self.stream = ctypes.c_void_p(stream)

    def __call__(self):
        st = self.lib.rog_gather_many(self.descs, self.n, self.W, self.stream)
        if st != 0:
            raise RuntimeError("rog_gather_many failed with status %d" % st)


def time_region(torch, fn, steps, warmup):
    """Elapsed ms of ``steps`` back-to-back calls, bracketed by synchronisation
    and two events on the calls' stream (the timed region)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def time_calls(torch, fn, steps, warmup):
    """Per-call event intervals (ms), as the pages time each call, and the
    elapsed ms of the whole sequence."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    region0.record()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    region1.record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in zip(starts, ends)], region0.elapsed_time(region1)


def to_device(torch, arrays, device):
    return [torch.from_numpy(a).to(device) for a in arrays]


def headline(torch, rog, wl, device, steps, warmup):
    case = wl.config4()
    payloads = [case.payload(r) for r in range(case.W)]
    srcs = to_device(torch, payloads, device)
    out = torch.empty(case.W * case.S, dtype=torch.uint8, device=device)
    plan = rog.rog_plan(srcs, out)
    call = Call(rog, srcs, out, torch.cuda.current_stream(device).cuda_stream)
    region_ms = time_region(torch, call, steps, warmup)
    per_call, _ = time_calls(torch, call, steps, 0)
    # Sampled parity of the timed launch configuration (first and last KiB of
    # every segment) against the definition.
    for r in range(case.W):
        for lo in (0, case.S - 1024):
            got = out[r * case.S + lo: r * case.S + lo + 1024].cpu().numpy()
            if not (got == payloads[r][lo:lo + 1024]).all():
                raise AssertionError("headline gather mismatch at rank %d offset %d" % (r, lo))
    return case, payloads, plan, per_call, region_ms, srcs


def misaligned(torch, rog, case, payloads, srcs, device, steps, warmup, in_off=1, out_off=3):
    """The headline payloads again, each at byte offset ``in_off`` of its own
    buffer, gathered to byte offset ``out_off``: the per-payload path with a
    16-byte body of aligned stores fed by unaligned loads.  Returns GB/s of the timed region and the plan."""
    views = []
    for s in srcs:
        buf = torch.empty(in_off + case.S, dtype=torch.uint8, device=device)
        buf[in_off:].copy_(s)
        views.append(buf[in_off:])
    obuf = torch.empty(out_off + case.W * case.S, dtype=torch.uint8, device=device)
    out = obuf[out_off:]
    plan = rog.rog_plan(views, out)
    region_ms = time_region(torch, Call(rog, views, out, torch.cuda.current_stream(device).cuda_stream),
                            steps, warmup)
    for r in range(case.W):
        for lo in (0, case.S - 1024):
            got = out[r * case.S + lo: r * case.S + lo + 1024].cpu().numpy()
            if not (got == payloads[r][lo:lo + 1024]).all():
                raise AssertionError("misaligned gather mismatch at rank %d offset %d" % (r, lo))
    return {"W": case.W, "bytes_per_rank": case.S, "src_offset": in_off, "out_offset": out_off,
            "kernel": plan["kernel"], "GBps": round(gbps(2 * case.W * case.S * steps, region_ms), 1),
            "ms_per_gather": round(region_ms / steps, 4)}


def latency_sweep(torch, rog, wl, device, steps=LATENCY_CALLS, warmup=LATENCY_WARMUP):
    """The two-payload case and the size sweep's 1 - 128 KiB payloads: every
    call event-timed (``steps`` calls after ``warmup``); p10 / p50 / p90, the
    number of calls and all samples (µs)."""
    rows = []
    cases = wl.config1() + [c for c in wl.config2() if c.S <= 128 * wl.KiB]
    stream = torch.cuda.current_stream(device).cuda_stream
    for case in cases:
        srcs = to_device(torch, [case.payload(r) for r in range(case.W)], device)
        out = torch.empty(case.W * case.S, dtype=torch.uint8, device=device)
        plan = rog.rog_plan(srcs, out)
        per_call, _ = time_calls(torch, Call(rog, srcs, out, stream), steps, warmup)
        s = summarize_ms(per_call)
        rows.append({"case": "c%d#%d" % (case.config, case.index), "W": case.W, "S_KiB": case.S // wl.KiB,
                     "path": plan["path"], "kernel": plan["kernel"],
                     "p10_us": round(s["p10_us"], 2), "p50_us": round(s["p50_us"], 2),
                     "p90_us": round(s["p90_us"], 2), "n": s["n"],
                     "eff_GBps": round(gbps(2 * case.W * case.S, s["p50_us"] * 1e-3), 1),
                     "samples_us": [round(1e3 * x, 2) for x in per_call]})
    return rows


def graph_latency(torch, rog, wl, device, per_graph=100):
    """Small gathers captured in a HIP graph: ``per_graph`` back-to-back calls per
    graph, replayed; the GPU time per gather with the host launch path removed."""
    rows = []
    cases = wl.config1() + [c for c in wl.config2() if c.S <= 128 * wl.KiB]
    for case in cases:
        srcs = to_device(torch, [case.payload(r) for r in range(case.W)], device)
        out = torch.empty(case.W * case.S, dtype=torch.uint8, device=device)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=device)
        side.wait_stream(torch.cuda.current_stream(device))
        with torch.cuda.stream(side):
            Call(rog, srcs, out, side.cuda_stream)()
        torch.cuda.current_stream(device).wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            call = Call(rog, srcs, out, torch.cuda.current_stream(device).cuda_stream)
            for _ in range(per_graph):
                call()
        per_replay, _ = time_calls(torch, g.replay, 10, 2)
        rows.append({"W": case.W, "S_KiB": case.S // wl.KiB,
                     "us_per_gather": round(1e3 * statistics.median(per_replay) / per_graph, 2)})
    return rows


def batch_bench(torch, rog, wl, device, steps, warmup):
    case = wl.config5(0)
    srcs = [to_device(torch, [case.payload(t, r) for r in range(case.W)], device)
            for t in range(len(case.tensors))]
    batch, outs = [], []
    for t, x in enumerate(case.tensors):
        # place every payload at its byte offset inside a slightly larger buffer
        views = []
        for s in srcs[t]:
            buf = torch.empty(x.in_off + x.S, dtype=torch.uint8, device=device)
            buf[x.in_off:].copy_(s)
            views.append(buf[x.in_off:])
        batch.append(views)
        ob = torch.empty(x.out_off + case.W * x.S, dtype=torch.uint8, device=device)
        outs.append(ob[x.out_off:])
    del srcs
    rog.rog_gather_many(batch, outs)           # checked once through the binding
    fn = BatchCall(rog, batch, outs, torch.cuda.current_stream(device).cuda_stream)
    per_call, _ = time_calls(torch, fn, steps, warmup)
    s = summarize_ms(per_call)
    moved = case.total_bytes_moved()
    odd = sum(1 for x in case.tensors if x.in_off or x.out_off)
    return {"W": case.W, "n": len(case.tensors), "odd_offset_tensors": odd, "bytes_moved": moved,
            "p50_us": round(s["p50_us"], 1), "GBps": round(gbps(moved, s["p50_us"] * 1e-3), 1)}


def d2d_ceiling(torch, device, nbytes, steps, warmup):
    a = torch.empty(nbytes, dtype=torch.uint8, device=device)
    b = torch.empty_like(a)
    per_call, _ = time_calls(torch, lambda: b.copy_(a), steps, warmup)
    return {"bytes": nbytes, "GBps": round(gbps(2 * nbytes, statistics.median(per_call)), 1),
            "how": "torch copy_ of one contiguous buffer (hipMemcpyAsync device to device)"}


# Untimed calls before the batched legs (3.2 and 5.1 GB moved per call): over
# freshly filled buffers the first 20-40 such calls run up to 10 % slower
# than the steady state the timed calls are meant to see.
BATCH_WARMUP = 40
BATCH_STEPS = 20

SWEEP_OUT_MIB = (64, 128, 256, 512)
SWEEP_CALLS = 40               # timed calls per case of the 64 - 512 MiB sweep (at least two passes over the sets)
SWEEP_MID_OUT_MIB = (2, 8, 32)
SWEEP_FOOTPRINT = 2 << 30      # bytes of rotating buffer sets per cold case (8 x the 256 MB cache)


def bandwidth_sweep(torch, rog, device, calls, out_mib=SWEEP_OUT_MIB, footprint=SWEEP_FOOTPRINT, graph=False,
                    ws=(2, 8), offsets=(0, 0)):
    """Gathers with outputs of ``out_mib`` (64 - 512 MiB by default, the
    "outputs >= 64 MiB" of the headline target) at each W of ``ws``, aligned
    or with every source and the output at the byte ``offsets`` (source,
    output) of their buffers, timed two ways over the same number of
    back-to-back launches (``calls``, or two passes over the sets if that is
    more): warm, the same buffers every call (as the pages time a call), and
    cold, rotating through K buffer sets that together span ``footprint``
    bytes, so that no call finds its sources in the 256 MB Infinity Cache.
    With ``graph`` the launches are captured into a HIP graph and the replay is
    timed, which takes the host's launch path (about 3.5 µs a call from Python,
    more than a small gather's kernel) out of the interval.  Sampled bytes of
    every set are checked against its sources."""
    src_off, out_off = offsets
    lib = rog.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    g = torch.Generator(device=device)
    g.manual_seed(20260)
    rows = []
    for W in ws:
        for mib in out_mib:
            S = (mib << 20) // W
            K = max(1, footprint // (2 * W * S))
            sets = []
            for _ in range(K):
                srcs = [torch.randint(0, 256, (S + src_off,), dtype=torch.uint8, device=device,
                                      generator=g)[src_off:] for _ in range(W)]
                out = torch.empty(W * S + out_off, dtype=torch.uint8, device=device)[out_off:]
                sets.append((srcs, out, (ctypes.c_void_p * W)(*[x.data_ptr() for x in srcs]),
                             ctypes.c_void_p(out.data_ptr())))

            def run(seq):
                for _, _, ptrs, o in seq[:K + 1]:
                    if lib.rog_gather(ptrs, W, S, o, stream) != 0:
                        raise RuntimeError("rog_gather failed")
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                if not graph:
                    e0.record()
                    for _, _, ptrs, o in seq:
                        lib.rog_gather(ptrs, W, S, o, stream)
                    e1.record()
                    torch.cuda.synchronize()
                    return e0.elapsed_time(e1) / len(seq)
                gr = torch.cuda.CUDAGraph()
                side = torch.cuda.Stream(device=device)
                side.wait_stream(torch.cuda.current_stream(device))
                with torch.cuda.graph(gr, stream=side):
                    sp = ctypes.c_void_p(side.cuda_stream)
                    for _, _, ptrs, o in seq:
                        if lib.rog_gather(ptrs, W, S, o, sp) != 0:
                            raise RuntimeError("rog_gather failed under capture")
                gr.replay()
                torch.cuda.synchronize()
                e0.record()
                gr.replay()
                e1.record()
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) / len(seq)

            n_calls = max(calls, 2 * K)
            warm_ms = run([sets[0]] * n_calls)
            cold_ms = run([sets[i % K] for i in range(n_calls)])
            for srcs, out, _, _ in sets:
                for r in range(W):
                    for lo in (0, S // 2, S - 1024):
                        if not torch.equal(out[r * S + lo: r * S + lo + 1024], srcs[r][lo:lo + 1024]):
                            raise AssertionError("sweep gather W=%d S=%d wrong at rank %d" % (W, S, r))
            moved = 2 * W * S
            kernel = rog.rog_plan(sets[0][0], sets[0][1])["kernel"]
            rows.append({"W": W, "out_MiB": mib, "offsets": list(offsets), "kernel": kernel, "sets": K, "calls": n_calls,
                         "timed": "graph replay" if graph else "eager launches",
                         "warm_GBps": round(gbps(moved, warm_ms), 1),
                         "warm_pct_of_peak": round(100 * gbps(moved, warm_ms) / PEAK_HBM_GBPS, 1),
                         "cold_GBps": round(gbps(moved, cold_ms), 1),
                         "cold_pct_of_peak": round(100 * gbps(moved, cold_ms) / PEAK_HBM_GBPS, 1),
                         "cold_us_per_gather": round(1e3 * cold_ms, 2)})
            del sets
            torch.cuda.empty_cache()
    return rows


def launch_floor(torch, device, steps=LATENCY_CALLS, warmup=LATENCY_WARMUP):
    """The eager floor of the per-call p50: one tiny torch kernel (a 1-element
    fill) issued from Python between the same two event records as a gather."""
    x = torch.empty(1, dtype=torch.int32, device=device)
    per_call, _ = time_calls(torch, x.zero_, steps, warmup)
    s = summarize_ms(per_call)
    return {"p10_us": round(s["p10_us"], 2), "p50_us": round(s["p50_us"], 2), "p90_us": round(s["p90_us"], 2),
            "n": s["n"], "how": "torch zero_ of a 1-element tensor, event-timed like the small gathers"}


CROSSOVER_TOTALS = (256, 1024, 4096, 8192, 16384, 32768, 40960, 49152, 65536, 81920, 98304,
                    114688, 131072, 262144, 1 << 20, 4 << 20)


def crossover(torch, rog, device, steps, warmup, totals=CROSSOVER_TOTALS):
    """Both forced paths on aligned outputs of the given sizes at W = 2 and 8,
    each call event-timed (the single-WG bound is chosen from these and from the
    kernel-only durations of the same command under rocprofv3 --kernel-trace).
    Call order per case: one checked call, ``warmup`` calls, ``steps`` timed
    calls; single-WG first, then multi-WG."""
    lib = rog.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    g = torch.Generator(device=device)
    g.manual_seed(7)
    rows = []
    for W in (2, 8):
        for total in totals:
            S = total // W
            srcs = [torch.randint(0, 256, (S,), dtype=torch.uint8, device=device, generator=g)
                    for _ in range(W)]
            out = torch.empty(total, dtype=torch.uint8, device=device)
            ptrs = (ctypes.c_void_p * W)(*[x.data_ptr() for x in srcs])
            o = ctypes.c_void_p(out.data_ptr())
            row = {"W": W, "output_bytes": total}
            for path, name in ((rog.ROG_PATH_SINGLE_WG, "single_wg"), (rog.ROG_PATH_MULTI_WG, "multi_wg")):
                call = lambda: lib.rog_gather_ex(ptrs, W, S, o, stream, path)  # noqa: E731
                out.zero_()
                if call() != 0:
                    raise RuntimeError("rog_gather_ex failed")
                torch.cuda.synchronize()
                if not torch.equal(out, torch.cat(srcs)):
                    raise AssertionError("crossover case W=%d total=%d path=%s is wrong" % (W, total, name))
                per_call, _ = time_calls(torch, call, steps, warmup)
                row[name + "_p50_us"] = round(1e3 * statistics.median(per_call), 2)
            rows.append(row)
            print(json.dumps(row), flush=True)
    return rows


# ---------------------------------------------------------------------------
# Rank-ordered sum (rog_reduce)
# ---------------------------------------------------------------------------

class ReduceCall:
    """A prepared rog_reduce_ex call: ctypes arguments built once."""

    def __init__(self, rog, srcs, out, stream, path=0):
        self.lib = rog.lib()
        self.W = len(srcs)
        self.n = srcs[0].numel()
        self.dtype = rog.DTYPES[srcs[0].dtype]
        self.ptrs = (ctypes.c_void_p * self.W)(*[s.data_ptr() for s in srcs])
        self.out = ctypes.c_void_p(out.data_ptr())
        self.stream = ctypes.c_void_p(stream)
        self.path = path

    def __call__(self):
        st = self.lib.rog_reduce_ex(self.ptrs, self.W, self.n, self.dtype, self.out, self.stream, self.path)
        if st != 0:
            raise RuntimeError("rog_reduce failed with status %d" % st)


def _reduce_tensors(torch, case, device):
    import numpy as np
    tdt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    payloads = case.payloads()
    srcs = [torch.from_numpy(p.view(np.int16) if case.dtype == "bf16" else p).to(device).view(tdt)
            for p in payloads]
    return payloads, srcs, torch.empty(case.n, dtype=tdt, device=device)


def reduce_bandwidth(torch, rog, wl, device, steps, warmup):
    """The rank-ordered sum of W = 8 bf16 payloads of 64 MiB: timed region and
    per-call p50.  Returns the result line, the payloads and the output (on the
    host) for the CPU-baseline leg, which checks a sample of it."""
    import numpy as np
    stream = torch.cuda.current_stream(device).cuda_stream
    case = wl.reduce_config4()
    payloads, srcs, out = _reduce_tensors(torch, case, device)
    call = ReduceCall(rog, srcs, out, stream)
    region_ms = time_region(torch, call, steps, warmup)
    per_call, _ = time_calls(torch, call, steps, 0)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    moved = (case.W + 1) * case.n * case.esize
    plan = rog.rog_reduce_plan(srcs, out)
    big = {"W": case.W, "dtype": case.dtype, "bytes_per_rank": case.n * case.esize, "bytes_moved": moved,
           "path": plan["path"], "grid": plan["grid"], "block": plan["block"],
           "mean_launch_us": round(1e3 * region_ms / steps, 2),
           "p50_us": round(1e3 * statistics.median(per_call), 2),
           "GBps": round(gbps(moved * steps, region_ms), 1),
           "pct_of_peak": round(100 * gbps(moved * steps, region_ms) / PEAK_HBM_GBPS, 2)}
    big["misaligned"] = reduce_misaligned(torch, rog, srcs, out, stream, steps, warmup)
    del srcs, out
    torch.cuda.empty_cache()
    return big, payloads, got


REDUCE_SWEEP_CASES = ((2, 0), (2, 1), (3, 0), (3, 1), (8, 0), (8, 1))   # (W, source element offset)
REDUCE_SWEEP_SOURCE_MIB = 512


def reduce_sweep(torch, rog, device, calls, footprint=SWEEP_FOOTPRINT):
    """Rank-ordered bf16 sums over 512 MiB of sources at W = 2, 3 and 8, the
    sources aligned with the output or one element off it, timed warm (the
    same buffers every call) and cold (rotating sets spanning ``footprint``
    bytes) over the same number of back-to-back launches, as the gather
    sweep is.  Each row records the launch's form (streamed loads, shared
    granules).  Sampled outputs are compared with a float32 sum in rank
    order, rounded once to bf16 (torch on the device), in every set."""
    lib = rog.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    g = torch.Generator(device=device)
    g.manual_seed(20261)
    rows = []
    for W, off in REDUCE_SWEEP_CASES:
        n = ((REDUCE_SWEEP_SOURCE_MIB << 20) // (2 * W)) // 64 * 64
        K = max(1, footprint // ((W + 1) * n * 2))
        sets = []
        for _ in range(K):
            bufs = [torch.randn(n + off, device=device, generator=g).to(torch.bfloat16) for _ in range(W)]
            srcs = [b[off:] for b in bufs]
            out = torch.empty(n, dtype=torch.bfloat16, device=device)
            sets.append((srcs, out, (ctypes.c_void_p * W)(*[x.data_ptr() for x in srcs]),
                         ctypes.c_void_p(out.data_ptr()), bufs))
        plan = rog.rog_reduce_plan(sets[0][0], sets[0][1])

        def run(seq):
            for _, _, ptrs, o, _ in (seq * 2)[:max(K + 1, 10)]:
                if lib.rog_reduce(ptrs, W, n, rog.ROG_DTYPE_BF16, o, stream) != 0:
                    raise RuntimeError("rog_reduce failed")
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _, _, ptrs, o, _ in seq:
                lib.rog_reduce(ptrs, W, n, rog.ROG_DTYPE_BF16, o, stream)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / len(seq)

        n_calls = max(calls, 2 * K)
        warm_ms = run([sets[0]] * n_calls)
        cold_ms = run([sets[i % K] for i in range(n_calls)])
        for srcs, out, _, _, _ in sets:
            for lo in (0, n // 2, n - 4096):
                acc = srcs[0][lo:lo + 4096].float()
                for r in range(1, W):
                    acc = acc + srcs[r][lo:lo + 4096].float()
                if not torch.equal(out[lo:lo + 4096].view(torch.int16), acc.to(torch.bfloat16).view(torch.int16)):
                    raise AssertionError("sweep sum W=%d offset %d wrong at element %d" % (W, off, lo))
        moved = (W + 1) * n * 2
        rows.append({"W": W, "source_MiB": W * n * 2 >> 20, "src_elem_offset": off, "sets": K, "calls": n_calls,
                     "nt_loads": plan["nt_loads"], "granules": plan["shifted_loads"],
                     "warm_GBps": round(gbps(moved, warm_ms), 1),
                     "warm_pct_of_peak": round(100 * gbps(moved, warm_ms) / PEAK_HBM_GBPS, 1),
                     "cold_GBps": round(gbps(moved, cold_ms), 1),
                     "cold_pct_of_peak": round(100 * gbps(moved, cold_ms) / PEAK_HBM_GBPS, 1)})
        del sets
        torch.cuda.empty_cache()
    return rows


SUM_PLACEMENT_CASES = (8, 3)                          # W
SUM_PLACEMENT_STRIDES = (None, 512, 128)              # None: one allocation per source
SUM_PLACEMENT_SOURCE_MIB = 64                         # per source


def sum_placements(torch, rog, device, calls=SWEEP_CALLS, footprint=SWEEP_FOOTPRINT):
    """The rank-ordered sum of W aligned bf16 sources of 64 MiB (W = 8 and 3)
    with the sources placed three ways: each in its own allocation (large
    allocations start on 2 MiB boundaries, so every source sits on the same
    128-byte place of a 1 KiB block), or carved from one allocation at strides
    of 64 MiB + 512 bytes (places alternating between two) or + 128 bytes
    (every source on its own place).  Timed warm (one set) and cold (rotating
    sets spanning ``footprint`` bytes) over the same number of back-to-back
    launches, as the other sweeps; sampled outputs of every set checked
    against a float32 sum in rank order rounded once to bf16."""
    lib = rog.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    g = torch.Generator(device=device)
    g.manual_seed(31337)
    n = (SUM_PLACEMENT_SOURCE_MIB << 20) // 2
    rows = []
    for W in SUM_PLACEMENT_CASES:
        K = max(2, footprint // ((W + 1) * n * 2))
        for stride in SUM_PLACEMENT_STRIDES:
            sets = []
            for _ in range(K):
                if stride is None:
                    keep = [torch.empty(n, dtype=torch.bfloat16, device=device) for _ in range(W)]
                    srcs = keep
                else:
                    step = 2 * n + stride
                    big = torch.empty(W * step, dtype=torch.uint8, device=device)
                    keep = [big]
                    srcs = [big[r * step: r * step + 2 * n].view(torch.bfloat16) for r in range(W)]
                for x in srcs:
                    x.copy_(torch.randn(n, device=device, generator=g))
                out = torch.empty(n, dtype=torch.bfloat16, device=device)
                sets.append((srcs, out, (ctypes.c_void_p * W)(*[x.data_ptr() for x in srcs]),
                             ctypes.c_void_p(out.data_ptr()), keep))
            places = [(x.data_ptr() >> 7) & 7 for x in sets[0][0]]

            def run(seq):
                for _, _, ptrs, o, _ in (seq * 2)[:max(K + 1, 10)]:
                    if lib.rog_reduce(ptrs, W, n, rog.ROG_DTYPE_BF16, o, stream) != 0:
                        raise RuntimeError("rog_reduce failed")
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _, _, ptrs, o, _ in seq:
                    lib.rog_reduce(ptrs, W, n, rog.ROG_DTYPE_BF16, o, stream)
                e1.record()
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) / len(seq)

            n_calls = max(calls, 2 * K)
            warm_ms = run([sets[0]] * n_calls)
            cold_ms = run([sets[i % K] for i in range(n_calls)])
            for srcs, out, _, _, _ in sets:
                for lo in (0, n // 2, n - 4096):
                    acc = srcs[0][lo:lo + 4096].float()
                    for r in range(1, W):
                        acc = acc + srcs[r][lo:lo + 4096].float()
                    if not torch.equal(out[lo:lo + 4096].view(torch.int16), acc.to(torch.bfloat16).view(torch.int16)):
                        raise AssertionError("placement sum W=%d stride %s wrong at element %d" % (W, stride, lo))
            moved = (W + 1) * n * 2
            rows.append({"W": W, "placement": "own allocations" if stride is None else "stride 64 MiB + %d B" % stride,
                         "line_places": places, "sets": K, "calls": n_calls,
                         "warm_GBps": round(gbps(moved, warm_ms), 1), "cold_GBps": round(gbps(moved, cold_ms), 1),
                         "cold_pct_of_peak": round(100 * gbps(moved, cold_ms) / PEAK_HBM_GBPS, 1)})
            del sets
            torch.cuda.empty_cache()
    return rows


CACHE_STATE_SETS = 4
CACHE_STATE_CALLS = 20
CACHE_STATE_PASS_BYTES = 1 << 30   # 4 x the 256 MB Infinity Cache


def cache_states(torch, rog, device, calls=CACHE_STATE_CALLS):
    """The headline gather (W = 8 x 64 MiB) and the rank-ordered sum of eight
    aligned bf16 payloads of 64 MiB, each in four cache states: back to back
    over one buffer set (as the headline is timed); back to back over four
    rotating sets (4.5 GiB for the gather, 2.3 GiB for the sum: no set's
    lines can still sit in the 256 MB Infinity Cache when it comes round
    again); and each call after a 1 GiB pass over other memory, read-only
    (the caches then hold clean lines of other data) or read-write (dirty
    lines, which the call's own cache allocations must write back first).
    The last two time each call alone, with events around it.  Every set's
    output is checked (gather: whole; sum: sampled against a float32 sum in
    rank order)."""
    lib = rog.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    g = torch.Generator(device=device)
    g.manual_seed(4044)
    scratch = torch.zeros(CACHE_STATE_PASS_BYTES // 8, dtype=torch.int64, device=device)
    sink = torch.empty(1, dtype=torch.int64, device=device)
    passes = {"after_read_pass": lambda: torch.sum(scratch, dim=0, keepdim=True, out=sink),
              "after_write_pass": lambda: scratch.add_(1)}

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def back_to_back(call, seq):
        for x in (seq * 2)[:len(seq) + CACHE_STATE_SETS]:
            call(x)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for x in seq:
            call(x)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / len(seq)

    def after_pass(call, x, pass_fn):
        call(x)
        total = 0.0
        for _ in range(calls):
            pass_fn()
            a, b = ev(), ev()
            a.record()
            call(x)
            b.record()
            torch.cuda.synchronize()
            total += a.elapsed_time(b)
        return total / calls

    def states(op, call, sets, moved):
        ms = {"back_to_back": back_to_back(call, [sets[0]] * calls),
              "rotating_%d_sets" % len(sets): back_to_back(call, [sets[i % len(sets)] for i in range(calls)])}
        for name, fn in passes.items():
            ms[name] = after_pass(call, sets[0], fn)
        base = gbps(moved, ms["back_to_back"])
        return [{"op": op, "state": k, "GBps": round(gbps(moved, v), 1),
                 "pct_of_peak": round(100 * gbps(moved, v) / PEAK_HBM_GBPS, 1),
                 "vs_back_to_back": round(gbps(moved, v) / base, 3)} for k, v in ms.items()]

    W, S = 8, 64 << 20
    sets = []
    for _ in range(CACHE_STATE_SETS):
        srcs = [torch.randint(0, 256, (S,), dtype=torch.uint8, device=device, generator=g) for _ in range(W)]
        out = torch.empty(W * S, dtype=torch.uint8, device=device)
        sets.append((srcs, out, (ctypes.c_void_p * W)(*[x.data_ptr() for x in srcs]), ctypes.c_void_p(out.data_ptr())))

    def gather(x):
        if lib.rog_gather(x[2], W, ctypes.c_size_t(S), x[3], stream) != 0:
            raise RuntimeError("rog_gather failed")

    rows = states("gather", gather, sets, 2 * W * S)
    for srcs, out, _, _ in sets:
        if not torch.equal(out, torch.cat(srcs)):
            raise AssertionError("cache-state gather wrong")
    del sets
    torch.cuda.empty_cache()

    n = S // 2
    sets = []
    for _ in range(CACHE_STATE_SETS):
        srcs = [torch.randn(n, device=device, generator=g).to(torch.bfloat16) for _ in range(W)]
        out = torch.empty(n, dtype=torch.bfloat16, device=device)
        sets.append((srcs, out, (ctypes.c_void_p * W)(*[x.data_ptr() for x in srcs]), ctypes.c_void_p(out.data_ptr())))

    def reduce(x):
        if lib.rog_reduce(x[2], W, ctypes.c_size_t(n), rog.ROG_DTYPE_BF16, x[3], stream) != 0:
            raise RuntimeError("rog_reduce failed")

    rows += states("sum", reduce, sets, (W + 1) * n * 2)
    for srcs, out, _, _ in sets:
        for lo in (0, n // 2, n - 4096):
            acc = srcs[0][lo:lo + 4096].float()
            for r in range(1, W):
                acc = acc + srcs[r][lo:lo + 4096].float()
            if not torch.equal(out[lo:lo + 4096].view(torch.int16), acc.to(torch.bfloat16).view(torch.int16)):
                raise AssertionError("cache-state sum wrong at element %d" % lo)
    del sets, scratch
    torch.cuda.empty_cache()
    return rows


def reduce_misaligned(torch, rog, srcs, aligned_out, stream, steps, warmup, in_off=1, out_off=0):
    """The same sum with every source at element offset ``in_off`` of its own
    buffer and the output at element offset ``out_off``: 2-byte source shifts,
    read as aligned granules shared between lanes.  Its output must equal the
    aligned sum's bit for bit."""
    n = aligned_out.numel()
    views = []
    for s in srcs:
        buf = torch.empty(in_off + n, dtype=s.dtype, device=s.device)
        buf[in_off:].copy_(s)
        views.append(buf[in_off:])
    obuf = torch.empty(out_off + n, dtype=aligned_out.dtype, device=aligned_out.device)
    out = obuf[out_off:]
    plan = rog.rog_reduce_plan(views, out)
    region_ms = time_region(torch, ReduceCall(rog, views, out, stream), steps, warmup)
    if not torch.equal(out.view(torch.int16), aligned_out.view(torch.int16)):
        raise AssertionError("the misaligned sum differs from the aligned one")
    moved = (len(srcs) + 1) * n * out.element_size()
    return {"src_elem_offset": in_off, "out_elem_offset": out_off, "shifted_loads": plan["shifted_loads"],
            "GBps": round(gbps(moved * steps, region_ms), 1), "mean_launch_us": round(1e3 * region_ms / steps, 2)}


def reduce_cpu_baseline(payloads, got, budget_s, sample=1 << 22, threads=None):
    """The CPU oracle on a bounded sample of the large sum (its first
    ``sample`` elements of all W payloads), repeated for about ``budget_s``
    seconds on one core and on every core this process may use (the oracle's
    sum called unchanged on element slices from a pool of threads); the sample
    of the GPU's output must equal it."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle
    T = threads or len(os.sched_getaffinity(0))
    srcs = [p[:sample] for p in payloads]
    want = np.empty(sample, np.uint16)
    oracle.reduce_c(srcs, want, "bf16")
    if not np.array_equal(got[:sample], want):
        raise AssertionError("the GPU's rank-ordered sum differs from the oracle's on the sample")
    reps1, el1 = repeat_for(lambda: oracle.reduce_c(srcs, want, "bf16"), budget_s)
    pieces = slices(sample, 4 * T)
    many = np.empty(sample, np.uint16)

    def piece(lohi):
        lo, hi = lohi
        oracle.reduce_c([s[lo:hi] for s in srcs], many[lo:hi], "bf16")

    with ThreadPoolExecutor(max_workers=T) as pool:
        list(pool.map(piece, pieces))
        repsT, elT = repeat_for(lambda: list(pool.map(piece, pieces)), budget_s)
    if not np.array_equal(many, want):
        raise AssertionError("the many-core oracle sum differs from the single-core one")
    moved = (len(srcs) + 1) * sample * 2
    return {"value": round(moved * repsT / elT / 1e9, 2), "unit": "GB/s", "cores": T, "kind": "oracle",
            "sample": "%d x the first %d elements of the W=%d bf16 sum (%.1f s) on %d threads, each calling "
                      "the C loop on slices of %d elements" % (repsT, sample, len(srcs), elT, T, sample // len(pieces)),
            "single_core": {"value": round(moved * reps1 / el1 / 1e9, 2), "unit": "GB/s", "cores": 1,
                            "sample": "%d x the same sample (%.1f s)" % (reps1, el1)}}


def reduce_latency(torch, rog, wl, device, steps=LATENCY_CALLS, warmup=LATENCY_WARMUP):
    """The pages' per-rank sizes 1 KiB - 4 MiB at W = 2 and 8: per-call p50 over
    ``steps`` event-timed calls."""
    stream = torch.cuda.current_stream(device).cuda_stream
    rows = []
    for c in wl.reduce_config2():
        _, srcs, out = _reduce_tensors(torch, c, device)
        p = rog.rog_reduce_plan(srcs, out)
        per_call, _ = time_calls(torch, ReduceCall(rog, srcs, out, stream), steps, warmup)
        sm = summarize_ms(per_call)
        rows.append({"W": c.W, "KiB_per_rank": c.n * c.esize // 1024, "path": p["path"],
                     "p10_us": round(sm["p10_us"], 2), "p50_us": round(sm["p50_us"], 2),
                     "p90_us": round(sm["p90_us"], 2), "n": sm["n"]})
    return rows


def reduce_batch(torch, rog, wl, device, steps, warmup):
    """rog_reduce_many over the batched gather's 16 tensor shapes (rows x cols
    bf16, W = 4) in one launch (the GPU tests check these shapes against the
    oracle)."""
    import numpy as np
    case = wl.config5(0)
    counts = [x.rows * x.cols for x in case.tensors]
    batch, outs = [], []
    for t, n in enumerate(counts):
        payloads = wl.reduce_payloads(wl.case_seed(26, t), case.W, n, "bf16")
        batch.append([torch.from_numpy(p.view(np.int16)).to(device).view(torch.bfloat16) for p in payloads])
        outs.append(torch.empty(n, dtype=torch.bfloat16, device=device))
    rog.rog_reduce_many(batch, outs)
    torch.cuda.synchronize()
    lib = rog.lib()
    keep = [(ctypes.c_void_p * case.W)(*[s.data_ptr() for s in srcs]) for srcs in batch]
    descs = (rog.rog_reduce_desc * len(batch))()
    for t, (o, n) in enumerate(zip(outs, counts)):
        descs[t].srcs = ctypes.cast(keep[t], ctypes.POINTER(ctypes.c_void_p))
        descs[t].out = ctypes.c_void_p(o.data_ptr())
        descs[t].count = n
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)

    def call():
        if lib.rog_reduce_many(descs, len(batch), case.W, rog.ROG_DTYPE_BF16, stream) != 0:
            raise RuntimeError("rog_reduce_many failed")
    per_call, _ = time_calls(torch, call, steps, warmup)
    moved = sum((case.W + 1) * n * 2 for n in counts)
    p50 = statistics.median(per_call)
    return {"W": case.W, "n": len(counts), "elements": sum(counts), "bytes_moved": moved,
            "p50_us": round(1e3 * p50, 1), "GBps": round(gbps(moved, p50), 1)}


REDUCE_CROSSOVER_KIB = (1, 2, 4, 8, 16, 24, 32, 48, 64, 128, 256)


def reduce_crossover(torch, rog, device, steps, warmup, sizes_kib=REDUCE_CROSSOVER_KIB):
    """Both forced paths of rog_reduce on bf16 outputs of the given sizes at W = 2
    and 8, each call event-timed (the bound is chosen from the kernel-only
    durations of the same command under rocprofv3 --kernel-trace).  Call order
    per case: one checked call, ``warmup`` calls, ``steps`` timed calls;
    single-WG first, then multi-WG."""
    stream = torch.cuda.current_stream(device).cuda_stream
    g = torch.Generator(device=device)
    g.manual_seed(8)
    rows = []
    for W in (2, 8):
        for kib in sizes_kib:
            n = kib * 512
            srcs = [(torch.rand(n, device=device, generator=g) * 2 - 1).to(torch.bfloat16) for _ in range(W)]
            outs = {}
            row = {"W": W, "output_bytes": 2 * n}
            for path, name in ((rog.ROG_PATH_SINGLE_WG, "single_wg"), (rog.ROG_PATH_MULTI_WG, "multi_wg")):
                out = torch.empty(n, dtype=torch.bfloat16, device=device)
                call = ReduceCall(rog, srcs, out, stream, path)
                call()
                torch.cuda.synchronize()
                outs[name] = out
                per_call, _ = time_calls(torch, call, steps, warmup)
                row[name + "_p50_us"] = round(1e3 * statistics.median(per_call), 2)
            if not torch.equal(outs["single_wg"].view(torch.int16), outs["multi_wg"].view(torch.int16)):
                raise AssertionError("reduce paths disagree at W=%d, %d KiB" % (W, kib))
            rows.append(row)
            print(json.dumps(row), flush=True)
    return rows


# hipDeviceAttribute_t values (hip_runtime_api.h): global memory bus width in
# bits, peak memory clock in kHz.
HIP_ATTR_MEMORY_BUS_WIDTH = 59
HIP_ATTR_MEMORY_CLOCK_RATE = 60


def hbm_from_runtime(device_index):
    """The HBM peak the HIP runtime's own figures imply, through the HIP
    runtime torch mapped: bus width x memory clock x transfers per clock.  On
    MI355X HIP reports 8192 bits and 2 GHz; two transfers per clock would give
    4.1 TB/s, less than the kernels here measure, so the figure takes four
    (8 Gb/s per pin, 8.2 TB/s: AMD's published 8 TB/s)."""
    from deterministic_collective_movement_amd import rog
    paths = sorted(rog._hip_runtimes_mapped())
    if len(paths) != 1:
        return {"error": "HIP runtimes mapped: %d" % len(paths)}
    hip = ctypes.CDLL(paths[0])
    vals = {}
    for name, attr in (("bus_width_bits", HIP_ATTR_MEMORY_BUS_WIDTH), ("memory_clock_khz", HIP_ATTR_MEMORY_CLOCK_RATE)):
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, device_index) != 0:
            return {"error": "hipDeviceGetAttribute(%d) failed" % attr}
        vals[name] = v.value
    vals["transfers_per_clock"] = 4
    vals["GBps"] = round(4 * vals["memory_clock_khz"] * 1e3 * vals["bus_width_bits"] / 8 / 1e9, 1)
    vals["denominator_used"] = "AMD's published %.0f GB/s, not this figure" % PEAK_HBM_GBPS
    return vals


def device_env(torch, device):
    """What the figures were measured on: the GPU's architecture name and
    compute-unit count, the HIP runtime's version, torch's own versions, and
    the digest of the gather kernels' sources the traffic figure is tied to."""
    env = {}
    try:
        props = torch.cuda.get_device_properties(device)
        env["gcn_arch"] = getattr(props, "gcnArchName", None)
        env["compute_units"] = props.multi_processor_count
        env["hbm_bytes"] = props.total_memory
    except Exception as e:   # the line is still printed without them
        env["device_error"] = str(e)
    try:
        from deterministic_collective_movement_amd import rog
        paths = sorted(rog._hip_runtimes_mapped())
        if len(paths) == 1:
            v = ctypes.c_int(0)
            if ctypes.CDLL(paths[0]).hipRuntimeGetVersion(ctypes.byref(v)) == 0:
                env["hip_runtime_version"] = v.value
    except Exception as e:
        env["hip_error"] = str(e)
    env["torch"] = torch.__version__
    env["torch_hip"] = getattr(torch.version, "hip", None)
    env["gather_kernel_sources_sha256"] = kernel_source_digest()
    return env


def host_cpu():
    """Model name and the number of cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "cores_available": len(os.sched_getaffinity(0))}


def slices(n, parts):
    """[lo, hi) pieces that cut range(n) into ``parts`` near-equal slices."""
    parts = max(1, min(parts, n))
    return [(n * k // parts, n * (k + 1) // parts) for k in range(parts)]


def repeat_for(fn, budget_s):
    """Call fn() until about budget_s seconds have passed; (calls, seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return reps, el


def cpu_baseline(case, payloads, budget_s, threads=None):
    """The CPU oracle on the full headline gather, repeated for about
    ``budget_s`` seconds: once on one core, once on every core this process
    may use.  The many-core form calls the oracle's gather unchanged on (payload,
    slice) pieces -- one payload per call, source and output pointers offset --
    from a pool of threads (the calls release the interpreter lock), so the
    bytes written are those of the single call.  The line reports the many-core
    figure, the single-core one beside it."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle
    T = threads or len(os.sched_getaffinity(0))
    S = case.S
    out = np.empty(case.W * S, np.uint8)
    oracle.gather_c(payloads, out)                  # untimed first touch of `out`
    reps1, el1 = repeat_for(lambda: oracle.gather_c(payloads, out), budget_s)
    per_payload = max(1, -(-4 * T // case.W))       # about 4 pieces per thread
    pieces = [(r, lo, hi) for r in range(case.W) for lo, hi in slices(S, per_payload)]

    def piece(job):
        r, lo, hi = job
        oracle.gather_c([payloads[r][lo:hi]], out[r * S + lo: r * S + hi])

    with ThreadPoolExecutor(max_workers=T) as pool:
        list(pool.map(piece, pieces))               # untimed warm-up of the pool
        repsT, elT = repeat_for(lambda: list(pool.map(piece, pieces)), budget_s)
    want = np.concatenate(payloads)
    if not np.array_equal(out, want):
        raise AssertionError("the many-core oracle gather differs from the concatenation")
    moved = 2 * case.W * S
    host = host_cpu()
    return {"value": round(moved * repsT / elT / 1e9, 2), "unit": "GB/s", "cores": T, "kind": "oracle",
            "sample": "%d x the full W=8 x 64 MiB gather (%.1f s) on %d threads, each calling the C per-byte "
                      "loop on (payload, slice) pieces of %d-%d bytes" % (repsT, elT, T, S // per_payload,
                                                                          -(-S // per_payload)),
            "cpu_model": host["model"], "cores_available": host["cores_available"],
            "single_core": {"value": round(moved * reps1 / el1 / 1e9, 2), "unit": "GB/s", "cores": 1,
                            "sample": "%d x the full gather (%.1f s), one call per gather" % (reps1, el1)}}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work")
    ap.add_argument("--no-native", action="store_true",
                    help="skip the C-timed small gathers (a child process), e.g. under a tracer")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline gather, its misaligned variant and the large "
                         "rank-ordered sum (for counter runs)")
    ap.add_argument("--calibrate-bytes", type=int, default=0,
                    help="also run a plain elementwise copy of this many bytes, for counter scaling")
    ap.add_argument("--reduce-crossover", action="store_true",
                    help="time both forced rog_reduce paths over small outputs instead")
    ap.add_argument("--crossover", action="store_true",
                    help="time both forced paths over small outputs instead (one JSON line per case)")
    ap.add_argument("--sweep-only", action="store_true",
                    help="time only the warm and cold bandwidth sweeps (2 - 512 MiB outputs), for traces")
    ap.add_argument("--reduce-sweep-only", action="store_true",
                    help="time only the rank-ordered sums' warm and cold sweep (W = 2, 3, 8), for counter runs")
    ap.add_argument("--cache-states-only", action="store_true",
                    help="time only the headline gather and W = 8 sum in the four cache states, for traces")
    ap.add_argument("--sum-placements-only", action="store_true",
                    help="time only the W = 8 and 3 sums with their sources placed three ways, for traces")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: --gpus %d is not supported (use --gpus 1)" % args.gpus,
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    from deterministic_collective_movement_amd import rog
    from deterministic_collective_movement_amd import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    if args.reduce_crossover:
        reduce_crossover(torch, rog, device, args.steps, args.warmup)
        return 0
    if args.crossover:
        crossover(torch, rog, device, args.steps, args.warmup)
        return 0
    if args.cache_states_only:
        print(json.dumps({"cache_states": cache_states(torch, rog, device)}), flush=True)
        return 0
    if args.sum_placements_only:
        print(json.dumps({"sum_placements": sum_placements(torch, rog, device)}), flush=True)
        return 0
    if args.reduce_sweep_only:
        print(json.dumps({"reduce_sweep": reduce_sweep(torch, rog, device, SWEEP_CALLS)}), flush=True)
        return 0
    if args.sweep_only:
        # eager launches throughout: under a kernel trace, graph-replayed
        # kernels carry the tracer's own cost per node
        print(json.dumps({"bandwidth_sweep": bandwidth_sweep(torch, rog, device, SWEEP_CALLS),
                          "bandwidth_sweep_mid": bandwidth_sweep(torch, rog, device, 50, out_mib=SWEEP_MID_OUT_MIB)}),
              flush=True)
        return 0

    case, payloads, plan, per_call, region_ms, srcs = headline(torch, rog, wl, device, args.steps, args.warmup)
    alg_bytes = 2 * case.W * case.S
    # Average launch duration of the headline kernel: the timed region's
    # back-to-back launches on one stream, divided by their number.
    mean_launch_ms = region_ms / args.steps
    value = gbps(alg_bytes * args.steps, region_ms)
    extras = {"headline": {"p50_us": round(1e3 * statistics.median(per_call), 2),
                           "mean_launch_us": round(1e3 * mean_launch_ms, 2),
                           "kernel": plan["kernel"], "path": plan["path"], "grid": plan["grid"],
                           "block": plan["block"],
                           "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2)}}
    if args.calibrate_bytes:
        a = torch.zeros(args.calibrate_bytes // 4, dtype=torch.int32, device=device)
        b = torch.empty_like(a)
        for _ in range(args.steps):
            torch.bitwise_not(a, out=b)
        torch.cuda.synchronize()
        extras["calibration"] = {"kernel": "torch.bitwise_not int32", "bytes_read": args.calibrate_bytes,
                                 "bytes_written": args.calibrate_bytes, "launches": args.steps}
    extras["misaligned"] = misaligned(torch, rog, case, payloads, srcs, device,
                                      max(10, args.steps // 5), max(2, args.warmup // 5))
    if not args.headline_only:
        extras["latency"] = latency_sweep(torch, rog, wl, device)
        extras["latency_floor"] = launch_floor(torch, device)
        extras["latency_native"] = {"skipped": "--no-native"} if args.no_native else latency_native()
        extras["latency_in_graph"] = graph_latency(torch, rog, wl, device)
        extras["gather_many"] = batch_bench(torch, rog, wl, device, BATCH_STEPS,
                                            max(BATCH_WARMUP, args.warmup))
        extras["d2d_copy_ceiling"] = d2d_ceiling(torch, device, case.W * case.S, 20, 3)
        extras["bandwidth_sweep"] = bandwidth_sweep(torch, rog, device, SWEEP_CALLS)
        if not args.no_native:
            # the empty launch's cost back to back (graph replay, grids of up to
            # 1024 workgroups) bounds what any one launch per gather can reach
            floor = launch_floor_native()
            null = [x["graph_us_per_launch"] for x in floor if x["kernel"] == "null" and x["grid"] <= 1024] \
                if isinstance(floor, list) else []
            extras["bandwidth_sweep_bound"] = (one_launch_bound(extras["bandwidth_sweep"], statistics.median(null))
                                               if null else {"error": floor.get("error", "no null rows")
                                                             if isinstance(floor, dict) else "no null rows"})
        # the same at byte offsets 1 (sources) and 3 (output): the PEER kernel
        extras["bandwidth_sweep_misaligned"] = bandwidth_sweep(torch, rog, device, SWEEP_CALLS, ws=(8,),
                                                               offsets=(1, 3))
        # the size sweep's 1 and 4 MiB payloads (outputs of 2 - 32 MiB), warm and cold
        extras["bandwidth_sweep_mid"] = bandwidth_sweep(torch, rog, device, 50, out_mib=SWEEP_MID_OUT_MIB,
                                                        graph=True)
        big, rpayloads, rgot = reduce_bandwidth(torch, rog, wl, device, args.steps, args.warmup)
        extras["reduce"] = {"bandwidth": big,
                            "sweep": reduce_sweep(torch, rog, device, SWEEP_CALLS),
                            "latency": reduce_latency(torch, rog, wl, device),
                            "batched": reduce_batch(torch, rog, wl, device, BATCH_STEPS,
                                                    max(BATCH_WARMUP, args.warmup))}
        extras["reduce"]["placements"] = sum_placements(torch, rog, device)
        extras["cache_states"] = cache_states(torch, rog, device)
        cpu = cpu_baseline(case, payloads, args.cpu_budget / 2)
        extras["reduce"]["cpu_baseline"] = reduce_cpu_baseline(rpayloads, rgot, min(2.5, args.cpu_budget / 4))
        del rpayloads, rgot
    else:
        extras["reduce"] = {"bandwidth": reduce_bandwidth(torch, rog, wl, device, max(10, args.steps // 2),
                                                          max(2, args.warmup // 2))[0]}
        cpu = None
    extras["device"] = torch.cuda.get_device_name(device)
    extras["env"] = device_env(torch, device)
    extras["hbm_from_runtime"] = hbm_from_runtime(device.index or 0)
    config = {"workload": "rank-ordered gather of W=8 aligned bf16 payloads of 64 MiB into a 512 MiB "
                          "output (1 GiB moved per step)",
              "W": case.W, "bytes_per_rank": case.S, "bytes_moved_per_step": alg_bytes}
    line = build_line(value=value, steps=args.steps, warmup=args.warmup, ms_per_step=region_ms / args.steps,
                      config=config, roof=roofline(alg_bytes, mean_launch_ms, read_traffic()),
                      cpu=cpu, extras=extras)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
