"""rog_gather, rog_gather_many and rog_reduce inside a captured HIP graph.

Each call is one kernel launch on the caller's stream with every argument in
the kernel arguments -- no allocation, no memset, no synchronisation -- so a
graph captures it as one kernel node.  The graph is replayed several times
with eager work and synchronisation between replays; the sources change
between replays, and every replay is checked against the CPU oracle for the
sources of that moment.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from deterministic_collective_movement_amd import rog
from deterministic_collective_movement_amd import workloads as wl
from oracle import oracle

pytestmark = pytest.mark.gpu


def _expected(srcs_dev):
    payloads = [s.cpu().numpy() for s in srcs_dev]
    out = np.empty(sum(p.shape[0] for p in payloads), np.uint8)
    oracle.gather_c(payloads, out)
    return out


def test_graph_replays_follow_the_current_sources(gpu):
    torch.cuda.synchronize()
    # three gathers of different classes: flat single-WG, per-peer, flat multi-WG
    specs = [(2, 1024, 0, 0), (3, 4095, 1, 3), (8, 128 * 1024, 0, 0)]
    cases = []
    for W, S, io, oo in specs:
        bufs = [torch.zeros(S + io + 16, dtype=torch.uint8, device=gpu) for _ in range(W)]
        srcs = [b[io:io + S] for b in bufs]
        ob = torch.full((W * S + oo + 16,), 0xA5, dtype=torch.uint8, device=gpu)
        cases.append((srcs, ob, ob[oo:oo + W * S], oo))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=gpu)
    side.wait_stream(torch.cuda.current_stream(gpu))
    with torch.cuda.stream(side):
        for srcs, _, out, _ in cases:          # warm-up outside the capture
            rog.rog_gather(srcs, out)
    torch.cuda.current_stream(gpu).wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for srcs, _, out, _ in cases:
            rog.rog_gather(srcs, out)
    rng = np.random.default_rng(5)
    for replay in range(4):
        # eager work between replays: new source bytes, and the outputs reset
        for srcs, ob, _, _ in cases:
            for s in srcs:
                s.copy_(torch.from_numpy(np.frombuffer(rng.bytes(s.numel()), np.uint8).copy()).to(gpu))
            ob.fill_(0xA5)
        torch.cuda.synchronize()
        print("graph replay %d" % replay, flush=True)
        g.replay()
        torch.cuda.synchronize()
        for srcs, ob, out, oo in cases:
            got = ob.cpu().numpy()
            assert np.array_equal(got[oo:oo + out.numel()], _expected(srcs)), (replay, len(srcs))
            assert np.all(got[:oo] == 0xA5) and np.all(got[oo + out.numel():] == 0xA5)


def test_graph_captures_a_batched_gather(gpu):
    case = wl.config5(3, n=6, W=4, max_rows=64)
    batch, outs, bufs = [], [], []
    for t, x in enumerate(case.tensors):
        srcs = []
        for r in range(case.W):
            b = torch.from_numpy(case.payload(t, r)).to(gpu)
            buf = torch.empty(x.in_off + x.S, dtype=torch.uint8, device=gpu)
            buf[x.in_off:].copy_(b)
            srcs.append(buf[x.in_off:])
        batch.append(srcs)
        ob = torch.empty(x.out_off + case.W * x.S, dtype=torch.uint8, device=gpu)
        outs.append(ob[x.out_off:])
    rog.rog_gather_many(batch, outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rog.rog_gather_many(batch, outs)
    for replay in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for srcs, o in zip(batch, outs):
            assert np.array_equal(o.cpu().numpy(), _expected(srcs)), replay


def test_graph_captures_rank_ordered_sums(gpu):
    """rog_reduce on both paths (single-WG and multi-WG), bf16 and binary32, in
    one captured graph; the sources change between replays and every replay
    matches the oracle bit for bit."""
    specs = [(2, 1000, "bf16"), (8, 70_001, "bf16"), (3, 40_000, "f32")]
    cases = []
    for W, n, dt in specs:
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        srcs = [torch.zeros(n, dtype=tdt, device=gpu) for _ in range(W)]
        cases.append((W, n, dt, srcs, torch.zeros(n, dtype=tdt, device=gpu)))
    for _, _, _, srcs, out in cases:
        rog.rog_reduce(srcs, out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, _, _, srcs, out in cases:
            rog.rog_reduce(srcs, out)
    for replay in range(4):
        wants = []
        for W, n, dt, srcs, out in cases:
            payloads = wl.reduce_payloads(wl.case_seed(20, replay * 10 + W), W, n, dt)
            for s, p in zip(srcs, payloads):
                s.copy_(torch.from_numpy(p.view(np.int16) if dt == "bf16" else p).to(gpu).view(s.dtype))
            out.zero_()
            want = np.empty(n, oracle.REDUCE_DTYPES[dt])
            oracle.reduce_c(payloads, want, dt)
            wants.append(want)
        torch.cuda.synchronize()
        print("graph replay %d (sums)" % replay, flush=True)
        g.replay()
        torch.cuda.synchronize()
        for (W, n, dt, _, out), want in zip(cases, wants):
            bits = torch.int16 if dt == "bf16" else torch.int32
            got = out.view(bits).cpu().numpy().view(want.dtype)
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (replay, W, n, dt)


def test_graph_captures_a_batched_sum(gpu):
    W = 3
    counts = [5, 4097, 30_000, 0, 123_457]
    batch = [[torch.zeros(n, dtype=torch.bfloat16, device=gpu) for _ in range(W)] for n in counts]
    outs = [torch.zeros(n, dtype=torch.bfloat16, device=gpu) for n in counts]
    rog.rog_reduce_many(batch, outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rog.rog_reduce_many(batch, outs)
    for replay in range(3):
        wants = []
        for t, (srcs, n) in enumerate(zip(batch, counts)):
            payloads = wl.reduce_payloads(wl.case_seed(25, replay * 10 + t), W, n, "bf16")
            for s, p in zip(srcs, payloads):
                s.copy_(torch.from_numpy(p.view(np.int16)).to(gpu).view(torch.bfloat16))
            want = np.empty(n, np.uint16)
            oracle.reduce_c(payloads, want, "bf16")
            wants.append(want)
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, want in zip(outs, wants):
            assert np.array_equal(o.view(torch.int16).cpu().numpy().view(np.uint16), want), replay


def test_graph_captures_streamed_forms(gpu):
    """The streamed-load forms in one graph: a 384 MiB sum at element offsets
    (granule form, lane shuffles) and a 384 MiB gather at byte offsets 1 / 3
    (shuffled PEER body); sources change between replays, every replay
    against the oracle."""
    W, n = 8, 24 << 20
    S = 2 * n + 3
    sum_bufs = [torch.zeros(n + 1, dtype=torch.bfloat16, device=gpu) for _ in range(W)]
    sum_srcs = [b[1:] for b in sum_bufs]
    sum_out = torch.zeros(n, dtype=torch.bfloat16, device=gpu)
    g_bufs = [torch.zeros(S + 1, dtype=torch.uint8, device=gpu) for _ in range(W)]
    g_srcs = [b[1:] for b in g_bufs]
    g_obuf = torch.zeros(W * S + 3, dtype=torch.uint8, device=gpu)
    g_out = g_obuf[3:]
    assert rog.rog_reduce_plan(sum_srcs, sum_out)["shifted_loads"]
    assert rog.rog_plan(g_srcs, g_out)["shifted_loads"]
    rog.rog_reduce(sum_srcs, sum_out)
    rog.rog_gather(g_srcs, g_out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rog.rog_reduce(sum_srcs, sum_out)
        rog.rog_gather(g_srcs, g_out)
    rng = np.random.default_rng(91)
    for replay in range(3):
        payloads = wl.reduce_payloads(wl.case_seed(27, replay), W, n, "bf16")
        for s, p in zip(sum_srcs, payloads):
            s.copy_(torch.from_numpy(p.view(np.int16)).to(gpu).view(torch.bfloat16))
        want_sum = np.empty(n, np.uint16)
        oracle.reduce_c(payloads, want_sum, "bf16")
        gp = [np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)]
        for s, p in zip(g_srcs, gp):
            s.copy_(torch.from_numpy(p).to(gpu))
        sum_out.zero_()
        g_out.zero_()
        torch.cuda.synchronize()
        print("graph replay %d (streamed forms)" % replay, flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(sum_out.view(torch.int16).cpu().numpy().view(np.uint16), want_sum), replay
        want_g = np.empty(W * S, np.uint8)
        oracle.gather_c(gp, want_g)
        assert np.array_equal(g_out.cpu().numpy(), want_g), replay
