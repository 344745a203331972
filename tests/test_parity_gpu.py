"""GPU parity: the HIP path through the C ABI against the CPU oracle, every byte
of every guarded buffer, on every forced path (auto, single-WG, multi-WG).

Cases are the workloads of the pages (RL-Align/RL-Kernel PR #491 "Results" and
"Tests"): the 2-payload 1 KiB gather, the size sweep at 2 and 8 payloads, the
alignment/tail sweep with odd offsets, the 8 x 64 MiB bandwidth case, the
batched gather, the pages' own size-test sizes, and edge cases (empty,
single payload, the maximum W, in place, aliased sources, payload boundaries
inside a wave's chunk).
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from deterministic_collective_movement_amd import rog
from deterministic_collective_movement_amd import workloads as wl
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_config1_two_1k_payloads(gpu):
    (case,) = wl.config1()
    gc.run_all_paths(gc.place_case(case, gpu), case.label())


@pytest.mark.parametrize("case", wl.config2(), ids=lambda c: c.label())
def test_config2_size_sweep(gpu, case):
    gc.run_all_paths(gc.place_case(case, gpu), case.label())


@pytest.mark.parametrize("case", wl.config3(), ids=lambda c: c.label())
def test_config3_alignment_and_tails(gpu, case):
    placed = gc.place_case(case, gpu)
    gc.run_all_paths(placed, case.label())


def test_config4_bandwidth_case_full_output(gpu):
    case = wl.config4()
    placed = gc.place_case(case, gpu)
    plan = rog.rog_plan(placed.srcs, placed.out)
    assert plan["kernel"] == "flat" and plan["path"] == "multi_wg"
    gc.run_all_paths(placed, case.label())


def test_config5_batched_one_launch(gpu):
    case = wl.config5(0)
    gc.place_batch(case, gpu).run("c5#0 W=4 n=16")


@pytest.mark.parametrize("index", range(1, 9))
def test_batched_small_mixes(gpu, index):
    """Batches of small tensors: flat and per-peer tensors side by side, empty
    tensors, W in {1, 3, 4, 8}."""
    W = (1, 3, 4, 8)[index % 4]
    case = wl.config5(index, n=12, W=W, max_rows=40)
    pb = gc.place_batch(case, gpu)
    pb.run("c5#%d small W=%d" % (index, W))


def test_batched_with_empty_tensors_and_mixed_sizes(gpu):
    rng = np.random.default_rng(17)
    W = 3
    sizes = [0, 16, 1, 4096, 0, 17, 65536, 255, 0]
    payloads = [[np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)] for S in sizes]
    in_offs = [0, 0, 3, 0, 1, 8, 0, 1, 0]
    out_offs = [0, 0, 1, 8, 0, 8, 0, 3, 5]
    gc.PlacedBatch(W, payloads, in_offs, out_offs, gpu).run("batch mixed")


def test_batched_maximum_batch(gpu):
    n = rog.rog_max_batch()
    W = rog.rog_max_batch_pointers() // n
    rng = np.random.default_rng(23)
    sizes = [int(rng.integers(1, 3000)) * 16 + (t % 3) for t in range(n)]
    payloads = [[np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)] for S in sizes]
    gc.PlacedBatch(W, payloads, [t % 2 for t in range(n)], [0] * n, gpu).run("batch max n=%d W=%d" % (n, W))


def _page_sizes():
    out = []
    with open(os.path.join(GOLDEN, "page_sizes.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(int(line))
    return out


@pytest.mark.parametrize("W", (2, 8))
@pytest.mark.parametrize("S", _page_sizes())
@pytest.mark.parametrize("offs", [(0, 0), (1, 3), (8, 8)])
def test_page_test_sizes(gpu, W, S, offs):
    case = wl.GatherCase(6, S * 10 + W, W, S, (offs[0],) * W, offs[1])
    gc.run_all_paths(gc.place_case(case, gpu), case.label())


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------

def test_zero_bytes_writes_nothing(gpu):
    placed = gc.Placed([np.zeros(0, np.uint8)] * 3, [0, 1, 2], 3, gpu)
    gc.run_all_paths(placed, "S=0")


@pytest.mark.parametrize("S", [1, 16, 1000, 4096, 1 << 20])
def test_single_payload_is_a_copy(gpu, S):
    case = wl.GatherCase(7, S, 1, S, (0,), 0)
    gc.run_all_paths(gc.place_case(case, gpu), case.label())


@pytest.mark.parametrize("S", [1, 15, 16, 48, 4096 + 3])
def test_maximum_W(gpu, S):
    W = rog.rog_max_peers()
    case = wl.GatherCase(8, S, W, S, tuple(r % 4 for r in range(W)) if S % 16 else (0,) * W, 0)
    gc.run_all_paths(gc.place_case(case, gpu), case.label())


@pytest.mark.parametrize("W,vpr", [(8, 1), (64, 1), (5, 3), (3, 255), (3, 257), (7, 1000), (2, 64 * 4 * 4 + 1)])
def test_payload_boundaries_inside_wave_chunks(gpu, W, vpr):
    """FLAT: payloads of vpr vectors, so chunks of 64*U vectors straddle one or
    many payload boundaries."""
    S = 16 * vpr
    payloads = [wl.tagged_payload(r, S) for r in range(W)]
    placed = gc.Placed(payloads, [0] * W, 0, gpu)
    assert rog.rog_plan(placed.srcs, placed.out)["kernel"] == "flat"
    gc.run_all_paths(placed, "tagged W=%d vpr=%d" % (W, vpr))


@pytest.mark.parametrize("W", [8, 9, 12, 16, 33, 64])
@pytest.mark.parametrize("S", [1024, 16 * 1000, 65536 + 16])
def test_flat_payloads_past_the_preloaded_pointers(gpu, W, S):
    """The multi-WG FLAT kernel holds the first eight payload pointers in
    scalar registers and reads the others from its arguments: tagged payloads
    on both sides of that boundary, chunks inside one payload and chunks
    across payloads, every byte against the oracle."""
    payloads = [wl.tagged_payload(r, S) for r in range(W)]
    placed = gc.Placed(payloads, [0] * W, 0, gpu)
    plan = rog.rog_plan(placed.srcs, placed.out, rog.ROG_PATH_MULTI_WG)
    assert plan["kernel"] == "flat" and plan["path"] == "multi_wg"
    gc.run_all_paths(placed, "tagged W=%d S=%d" % (W, S), paths=(rog.ROG_PATH_MULTI_WG,))


# Output offsets past the 64-byte guard: the output then sits 16 * k bytes past
# a 128-byte line for every k in 0..7, so the multi-WG FLAT kernel cuts its
# first chunk short by each possible shift.
LINE_OFFSETS = [(16 * k - wl.GUARD) % 128 for k in range(8)]


@pytest.mark.parametrize("W", [1, 3, 8])
@pytest.mark.parametrize("S", [16, 1024, 16 * 257, 65536 + 48, (1 << 20) + 16])
def test_flat_output_at_every_line_offset(gpu, W, S):
    """FLAT gathers whose output sits anywhere on the 128-byte line grid, with
    sources at other line offsets: the first chunk is short by the output's
    offset / 16 vectors and the rest start on lines; every byte, the guards
    and the sources against the oracle on every path."""
    payloads = [wl.tagged_payload(r + 5, S) for r in range(W)]
    for k, oo in enumerate(LINE_OFFSETS):
        offs = [(16 * (3 * r + k)) % 128 for r in range(W)]
        placed = gc.Placed(payloads, offs, oo, gpu)
        assert rog.rog_plan(placed.srcs, placed.out)["kernel"] == "flat"
        line = (placed.out.data_ptr() % 128) // 16
        gc.run_all_paths(placed, "flat W=%d S=%d out line offset %d srcs %s" % (W, S, 16 * line, offs))


def test_flat_batch_off_the_line_grid(gpu):
    """A batch mixing FLAT tensors on the line grid (round-robin group), FLAT
    tensors off it (shifted first chunk, XCD runs) and PEER tensors: every
    tensor against the oracle."""
    W = 3
    rng = np.random.default_rng(123)
    sizes = [4096, 16 * 1000, 65536, 48, (1 << 20) + 16, 1024, 4096 + 5, 16 * 77]
    in_offs = [64, 16, 64, 112, 0, 80, 3, 32]
    out_offs = [64, 80, 0, 16, 112, 64, 7, 48]
    payloads = [[np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)] for S in sizes]
    b = gc.PlacedBatch(W, payloads, in_offs, out_offs, gpu)
    lines = [((it.out.data_ptr() | it.S | it.srcs[0].data_ptr()) % 128 == 0) for it in b.items]
    assert any(lines) and not all(lines)
    b.run("flat batch off the line grid")


def test_streamed_flat_gather_off_the_line_grid(gpu):
    """FLAT with streamed loads (384 MiB of sources), output 16 bytes past a
    line and every source at its own line offset: every byte against the
    oracle."""
    S = 48 << 20
    rng = np.random.default_rng(321)
    payloads = [np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(8)]
    oo = (16 - wl.GUARD) % 128
    placed = gc.Placed(payloads, [(16 * r) % 128 for r in range(8)], oo, gpu)
    plan = rog.rog_plan(placed.srcs, placed.out)
    assert plan["kernel"] == "flat" and plan["path"] == "multi_wg" and plan["nt_loads"]
    assert placed.out.data_ptr() % 128 == 16
    gc.run_all_paths(placed, "streamed flat, out 16 past a line", paths=(rog.ROG_PATH_AUTO,))


@pytest.mark.parametrize("W,S,offs", [(2, 64 << 20, (0, 0)), (8, 16 << 20, (16, 48)), (4, (32 << 20) - 1024, (0, 0))],
                         ids=["2x64MiB", "8x16MiB_off_lines", "4x32MiB-1KiB"])
def test_flat_gathers_around_the_streaming_bound(gpu, W, S, offs):
    """FLAT gathers stream their loads from 128 MiB of sources: at the bound
    (2 x 64 MiB and, off the line grid, 8 x 16 MiB) and just below it (cached
    loads), every byte against the oracle."""
    rng = np.random.default_rng(W * 1000 + S % 997)
    payloads = [np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)]
    in_off, out_off = offs
    placed = gc.Placed(payloads, [(in_off - wl.GUARD) % 128] * W, (out_off - wl.GUARD) % 128, gpu)
    assert placed.out.data_ptr() % 128 == out_off and placed.srcs[0].data_ptr() % 128 == in_off
    plan = rog.rog_plan(placed.srcs, placed.out)
    assert plan["kernel"] == "flat" and plan["path"] == "multi_wg"
    assert plan["nt_loads"] is (W * S >= 128 << 20)
    gc.run_all_paths(placed, "flat %d x %d" % (W, S), paths=(rog.ROG_PATH_AUTO,))


@pytest.mark.parametrize("W,S,io,oo", [(8, (16 << 20) + 5, 1, 3), (8, (16 << 20) - 3, 1, 3),
                                        (2, (64 << 20) + 1, 0, 1), (4, 32 << 20, 2, 0)],
                         ids=["8x16MiB+5_at_1_3", "8x16MiB-3_at_1_3", "2x64MiB+1_at_0_1", "4x32MiB_at_2_0"])
def test_peer_gathers_around_the_streaming_bound(gpu, W, S, io, oo):
    """PEER gathers stream their loads from 128 MiB of sources, as FLAT ones
    do, and then read shifted sources as shared granules: just above the bound
    and just below it (cached, unaligned loads), every byte against the
    oracle."""
    rng = np.random.default_rng(W * 7919 + S % 1009 + io)
    payloads = [np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)]
    placed = gc.Placed(payloads, [io] * W, oo, gpu)
    plan = rog.rog_plan(placed.srcs, placed.out)
    assert plan["kernel"] == "peer" and plan["path"] == "multi_wg"
    assert plan["nt_loads"] is (W * S >= 128 << 20)
    assert plan["shifted_loads"] == (plan["nt_loads"] and _shares_granules(placed))
    gc.run_all_paths(placed, "peer %d x %d at (%d, %d)" % (W, S, io, oo), paths=(rog.ROG_PATH_AUTO,))


@pytest.mark.parametrize("S,W", [(16 * 1000, 4), (4095, 3), (1 << 20, 8)])
def test_exact_in_place_segments(gpu, S, W):
    """Payloads 1 and 3 already sit in their own output segments."""
    rng = np.random.default_rng(S + W)
    payloads = [np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)]
    placed = gc.Placed(payloads, [0] * W, 0, gpu)
    for path in gc.PATHS:
        placed.reset_output()
        srcs = list(placed.srcs)
        for r in (1, 3):
            if r < W:
                placed.out[r * S:(r + 1) * S].copy_(placed.srcs[r])
                srcs[r] = placed.out[r * S:(r + 1) * S]
        rog.rog_gather_ex(srcs, placed.out, path)
        placed.check("in place S=%d W=%d path=%d" % (S, W, path))


def test_aliased_sources(gpu):
    rng = np.random.default_rng(31)
    S = 12345
    p = np.frombuffer(rng.bytes(S), np.uint8).copy()
    placed = gc.Placed([p], [1], 0, gpu)
    out = torch.full((4 * S,), 0, dtype=torch.uint8, device=gpu)
    for path in gc.PATHS:
        out.zero_()
        rog.rog_gather_ex([placed.srcs[0]] * 4, out, path)
        torch.cuda.synchronize()
        assert out.cpu().numpy().tobytes() == p.tobytes() * 4


def test_returns_out_and_allocates_when_absent(gpu):
    a = torch.arange(64, dtype=torch.int16, device=gpu)
    b = -a
    out = rog.rog_gather([a, b])
    torch.cuda.synchronize()
    assert out.dtype == torch.uint8 and out.numel() == 256
    assert torch.equal(out.view(torch.int16), torch.cat([a, b]))
    o2 = torch.empty(128, dtype=torch.int16, device=gpu)
    assert rog.rog_gather([a, b], out=o2) is o2


def test_runs_on_the_given_stream(gpu):
    s = torch.cuda.Stream(device=gpu)
    a = torch.randint(0, 255, (1 << 20,), dtype=torch.uint8, device=gpu)
    b = torch.randint(0, 255, (1 << 20,), dtype=torch.uint8, device=gpu)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = rog.rog_gather([a, b])
    s.synchronize()
    assert torch.equal(out, torch.cat([a, b]))


def test_binding_rejects_bad_tensors(gpu):
    a = torch.zeros(16, dtype=torch.uint8, device=gpu)
    with pytest.raises(ValueError):
        rog.rog_gather([a, torch.zeros(17, dtype=torch.uint8, device=gpu)])
    with pytest.raises(ValueError):
        rog.rog_gather([a, a], out=torch.zeros(31, dtype=torch.uint8, device=gpu))
    with pytest.raises(ValueError):
        rog.rog_gather([a, torch.zeros(16, dtype=torch.uint8)])
    with pytest.raises(ValueError):
        rog.rog_gather([a, a], out=torch.zeros(64, dtype=torch.uint8, device=gpu)[::2])
    with pytest.raises(rog.RogArgumentError):
        buf = torch.zeros(64, dtype=torch.uint8, device=gpu)
        rog.rog_gather([buf[8:24], a], out=buf[0:32])


def test_largest_vector_index(gpu):
    """FLAT at the top of the 32-bit vector index: W*S just below 2^36 bytes.
    Checked at full size through properties that hold at any size: sampled
    windows at both ends of every segment, across payload boundaries and at the
    very end of the output equal the corresponding source bytes."""
    W = 8
    S = (1 << 33) - 16                     # 8 GiB - 16 per payload
    total = W * S                          # 2^36 - 128 bytes: n_vec = 2^32 - 8
    free, _ = torch.cuda.mem_get_info(gpu)
    if free < 2 * total + (8 << 30):
        pytest.skip("needs %d GiB of free device memory" % ((2 * total >> 30) + 8))
    srcs = []
    for r in range(W):
        t = torch.empty(S, dtype=torch.uint8, device=gpu)
        t.fill_(r * 29 + 7)
        srcs.append(t)
    rng = np.random.default_rng(99)
    win = 4096
    windows = [0, S - win, S // 2]
    for r in range(W):
        for lo in windows:
            srcs[r][lo:lo + win].copy_(torch.from_numpy(np.frombuffer(rng.bytes(win), np.uint8).copy()))
    out = torch.empty(total, dtype=torch.uint8, device=gpu)
    assert rog.rog_plan(srcs, out)["kernel"] == "flat"
    print("largest vector index W=8 S=%d" % S, flush=True)
    rog.rog_gather(srcs, out)
    torch.cuda.synchronize()
    for r in range(W):
        for lo in windows:
            got = out[r * S + lo: r * S + lo + win].cpu()
            want = srcs[r][lo:lo + win].cpu()
            assert torch.equal(got, want), (r, lo)
    # the filled stretches between windows carry the per-rank fill value
    for r in range(W):
        mid = out[r * S + win: r * S + win + (1 << 20)].cpu()
        assert torch.all(mid == r * 29 + 7)
    del out, srcs
    torch.cuda.empty_cache()


def test_largest_misaligned_gather(gpu):
    """PEER at the top of the size range: W = 8 payloads of 8 GiB - 21 bytes
    (W*S = 2^36 - 168) with the sources at byte offset 1 and the output at 3,
    so streamed loads and the lane shuffle.  Checked through properties that
    hold at any size: sampled windows at both ends and in the middle of every
    segment equal their source bytes, and the filled stretches between them
    carry the per-rank value."""
    W = 8
    S = (1 << 33) - 21
    total = W * S
    free, _ = torch.cuda.mem_get_info(gpu)
    if free < 2 * total + (8 << 30):
        pytest.skip("needs %d GiB of free device memory" % ((2 * total >> 30) + 8))
    bufs, srcs = [], []
    for r in range(W):
        t = torch.empty(S + 1, dtype=torch.uint8, device=gpu)
        t.fill_(r * 31 + 5)
        bufs.append(t)
        srcs.append(t[1:])
    rng = np.random.default_rng(98)
    win = 4096
    windows = [0, S - win, S // 2 + 7]
    for r in range(W):
        for lo in windows:
            srcs[r][lo:lo + win].copy_(torch.from_numpy(np.frombuffer(rng.bytes(win), np.uint8).copy()))
    obuf = torch.empty(total + 3, dtype=torch.uint8, device=gpu)
    out = obuf[3:]
    plan = rog.rog_plan(srcs, out)
    assert plan["kernel"] == "peer" and plan["path"] == "multi_wg" and plan["nt_loads"] and plan["shifted_loads"]
    print("largest misaligned gather W=8 S=%d" % S, flush=True)
    rog.rog_gather(srcs, out)
    torch.cuda.synchronize()
    for r in range(W):
        for lo in windows:
            assert torch.equal(out[r * S + lo: r * S + lo + win].cpu(), srcs[r][lo:lo + win].cpu()), (r, lo)
        mid = out[r * S + win: r * S + win + (1 << 20)].cpu()
        assert torch.all(mid == r * 31 + 5), r
    del out, obuf, srcs, bufs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("W", [1, 3])
def test_every_source_and_destination_misalignment(gpu, W):
    """The per-peer path's head / aligned body / tail cut for every pair of
    source and destination misalignments (mod 16), at sizes around the
    smallest payload with a body and at sizes with a long body, on every path.
    Payloads are peer-tagged, so a misplaced or shifted byte cannot hide."""
    sizes = (17, 47, 48, 49, 63, 64, 100, 1000, 70001)
    for so in range(16):
        for do in range(16):
            for S in sizes:
                payloads = [wl.tagged_payload(r + 3 * so, S) for r in range(W)]
                placed = gc.Placed(payloads, [so] * W, do, gpu)
                gc.run_all_paths(placed, "misaligned W=%d S=%d src%%16=%d dst%%16=%d" % (W, S, so, do))


def test_misaligned_large_payloads(gpu):
    """Multi-workgroup 1 KiB chunks of the body over payloads of 8 MiB + 5
    (32768 chunks: whole spans of XCD-grouped chunks)."""
    S = (8 << 20) + 5
    rng = np.random.default_rng(41)
    payloads = [np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(4)]
    for io, oo in [(1, 3), (3, 3), (0, 9), (15, 0)]:
        placed = gc.Placed(payloads, [io, io + 4, io, 8], oo, gpu)
        gc.run_all_paths(placed, "misaligned large in=%d out=%d" % (io, oo),
                         paths=(rog.ROG_PATH_AUTO, rog.ROG_PATH_MULTI_WG))


@pytest.mark.parametrize("W,S", [(5, (256 << 10) + 3), (3, (1 << 20) + 7), (7, 64 * 16 * 150 + 9)])
def test_chunk_counts_beyond_whole_xcd_spans(gpu, W, S):
    """Chunk counts that leave a remainder after the whole spans of XCD-grouped
    chunks (5 x 256 KiB+3: 1280 chunks = one span of 1024 + 256), or fill them
    exactly (3 x 1 MiB+7: 3072), or have no whole span (7 x 150 chunks); every
    payload peer-tagged and misaligned differently."""
    payloads = [wl.tagged_payload(r + 11, S) for r in range(W)]
    offs = [(3 * r + 1) % 16 for r in range(W)]
    placed = gc.Placed(payloads, offs, 5, gpu)
    gc.run_all_paths(placed, "chunk spans W=%d S=%d" % (W, S),
                     paths=(rog.ROG_PATH_AUTO, rog.ROG_PATH_MULTI_WG))


@pytest.fixture(scope="module")
def streamed_payloads():
    """8 payloads of 48 MiB + 5 bytes: 384 MiB of sources, enough for the
    kernels to stream their loads past the caches."""
    S = (48 << 20) + 5
    rng = np.random.default_rng(77)
    return [np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(8)]


def _shares_granules(placed):
    """The PEER kernel's rule for streamed loads: some payload's source sits an
    odd or 2-mod-4 number of bytes past a 16-byte granule where its body (from
    the first 256-byte boundary of its output) starts."""
    o = placed.out.data_ptr()
    for r, s in enumerate(placed.srcs):
        head = (256 - (o + r * placed.S) % 256) % 256
        if placed.S >= head + 16 and ((s.data_ptr() + head) % 16) % 4:
            return True
    return False


@pytest.mark.parametrize("io,oo", [(1, 3), (0, 1), (2, 0), (4, 0), (5, 5)])
def test_misaligned_streamed_payloads(gpu, streamed_payloads, io, oo):
    """Misaligned payloads with streamed loads, where the PEER body reads
    aligned granules shared between lanes at odd and 2-mod-4 shifts (and
    unaligned loads at the others): every byte against the oracle."""
    placed = gc.Placed(streamed_payloads, [io] * 8, oo, gpu)
    plan = rog.rog_plan(placed.srcs, placed.out)
    assert plan["kernel"] == "peer" and plan["path"] == "multi_wg" and plan["nt_loads"]
    assert plan["shifted_loads"] == _shares_granules(placed)
    gc.run_all_paths(placed, "streamed misaligned in=%d out=%d" % (io, oo), paths=(rog.ROG_PATH_AUTO,))


def test_streamed_payloads_each_misaligned_differently(gpu, streamed_payloads):
    placed = gc.Placed(streamed_payloads, list(range(1, 9)), 7, gpu)
    plan = rog.rog_plan(placed.srcs, placed.out)
    assert plan["nt_loads"] and plan["shifted_loads"]
    gc.run_all_paths(placed, "streamed misaligned, source offsets 1..8, out 7", paths=(rog.ROG_PATH_AUTO,))


def test_streamed_batch_with_small_misaligned_tensors(gpu):
    """A batch whose sources total 128 MiB or more streams its loads, so its
    misaligned tensors take the shuffled PEER body, down to tensors of a few
    bytes and bodies shorter than one wave: one 100 MiB tensor (W = 4) beside
    small and empty tensors at odd offsets."""
    rng = np.random.default_rng(88)
    W = 4
    sizes = [100 << 20, 0, 1, 17, 255, 256 + 5, 1040, 4096 + 3, 65536 + 7, 1 << 20]
    in_offs = [1, 0, 3, 1, 2, 1, 5, 3, 1, 2]
    out_offs = [3, 0, 0, 1, 0, 3, 7, 2, 9, 0]
    payloads = [[np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)] for S in sizes]
    gc.PlacedBatch(W, payloads, in_offs, out_offs, gpu).run("streamed batch, small misaligned tensors")


def test_streamed_batch_from_128_MiB(gpu):
    """A batch streams its loads from 128 MiB of sources, as a single gather
    does: 8 tensors of 6 MiB + 5 per payload (W = 4, 192 MiB of sources), at
    odd offsets (shuffled PEER bodies) beside aligned ones, every byte against
    the oracle."""
    rng = np.random.default_rng(91)
    W = 4
    sizes = [(6 << 20) + 5] * 4 + [6 << 20] * 4
    payloads = [[np.frombuffer(rng.bytes(S), np.uint8).copy() for _ in range(W)] for S in sizes]
    gc.PlacedBatch(W, payloads, [1, 3, 0, 2, 0, 0, 0, 0], [3, 1, 1, 0, 0, 0, 0, 0], gpu).run(
        "streamed batch of 192 MiB")
