"""The rank-ordered sum on the GPU against the CPU oracle, bit for bit (a NaN
matches any NaN), through the C ABI, on every path: the pages' per-rank sizes
across their 256 KiB single-block bound, element alignments and ragged tails,
random bit patterns (NaNs, infinities, subnormals), in place, aliased sources,
the largest W, and the full bandwidth case."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from deterministic_collective_movement_amd import rog
from deterministic_collective_movement_amd import workloads as wl
from oracle import oracle
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


def test_two_1k_payloads(gpu):
    case = wl.reduce_config1()[0]
    gc.run_reduce_all_paths(gc.place_reduce(case, gpu), case.label())


@pytest.mark.parametrize("case", wl.reduce_config2(), ids=lambda c: c.label())
def test_size_sweep(gpu, case):
    gc.run_reduce_all_paths(gc.place_reduce(case, gpu), case.label())


@pytest.mark.parametrize("case", wl.reduce_config3(), ids=lambda c: c.label())
def test_alignment_tails_and_bit_patterns(gpu, case):
    gc.run_reduce_all_paths(gc.place_reduce(case, gpu), case.label())


def test_bandwidth_case_full_output(gpu):
    """W = 8 bf16 payloads of 64 MiB: every element against the oracle."""
    case = wl.reduce_config4()
    placed = gc.place_reduce(case, gpu)
    plan = rog.rog_reduce_plan(placed.srcs, placed.out)
    assert plan["path"] == "multi_wg" and plan["nt_loads"]
    gc.run_reduce_all_paths(placed, case.label(), paths=(rog.ROG_PATH_AUTO,))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("W", [1, 5, 64])
def test_every_W_up_to_the_maximum(gpu, dtype, W):
    assert W <= rog.rog_max_peers()
    for n in (1, 1000, 70001):
        payloads = wl.reduce_payloads(wl.case_seed(15, W * 10 + n % 7), W, n, dtype)
        placed = gc.PlacedReduce(payloads, [r % 4 for r in range(W)], 3, dtype, gpu)
        gc.run_reduce_all_paths(placed, "W=%d n=%d %s" % (W, n, dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("which", [0, 2])
def test_in_place(gpu, dtype, which):
    """out is srcs[which] itself (an in-place all-reduce)."""
    n = 50_003
    payloads = wl.reduce_payloads(wl.case_seed(16, which), 3, n, dtype)
    placed = gc.PlacedReduce(payloads, [1, 0, 2], 0, dtype, gpu, in_place=which)
    gc.run_reduce_all_paths(placed, "in place srcs[%d] %s" % (which, dtype))


def test_aliased_sources(gpu):
    """The same buffer passed as several ranks: x + x + y, in that order."""
    n = 40_000
    x, y = wl.reduce_payloads(wl.case_seed(17, 0), 2, n, "bf16")
    placed = gc.PlacedReduce([x, y], [0, 0], 0, "bf16", gpu)
    srcs = [placed.srcs[0], placed.srcs[0], placed.srcs[1]]
    want = np.empty(n, np.uint16)
    oracle.reduce_c([x, x, y], want, "bf16")
    for path in gc.PATHS:
        placed.reset()
        rog.rog_reduce_ex(srcs, placed.out, path)
        torch.cuda.synchronize()
        got = placed.out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), rog.PATH_NAMES[path]


def test_repeated_calls_give_identical_bits(gpu):
    """Determinism: the same call on both paths, many times, the same bits."""
    n = 1 << 20
    payloads = wl.reduce_payloads(wl.case_seed(18, 0), 8, n, "bf16")
    placed = gc.PlacedReduce(payloads, [0] * 8, 0, "bf16", gpu)
    outs = []
    for k in range(10):
        path = (rog.ROG_PATH_MULTI_WG, rog.ROG_PATH_SINGLE_WG)[k % 2]
        outs.append(rog.rog_reduce_ex(placed.srcs, None, path))
    torch.cuda.synchronize()
    first = outs[0].view(torch.int16)
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), first)
    placed.reset()
    rog.rog_reduce(placed.srcs, placed.out)
    placed.check("determinism reference")


def test_reduce_scatter_shares(gpu):
    """rog_reduce_scatter: rank r gets the sum of every input's shard r."""
    W, n = 4, 12_345
    inputs = wl.reduce_payloads(wl.case_seed(19, 0), W, W * n, "f32")
    dev = [torch.from_numpy(x).to(gpu) for x in inputs]
    for rank in range(W):
        got = rog.rog_reduce_scatter(dev, rank)
        want = np.empty(n, np.float32)
        oracle.reduce_c([x[rank * n:(rank + 1) * n] for x in inputs], want, "f32")
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32)), rank


def test_zero_elements_writes_nothing(gpu):
    placed = gc.PlacedReduce([np.zeros(0, np.float32)] * 2, [0, 0], 0, "f32", gpu)
    rog.rog_reduce(placed.srcs, placed.out)
    placed.check("n = 0")


def test_binding_rejects_bad_tensors(gpu):
    a = torch.zeros(16, dtype=torch.float32, device=gpu)
    with pytest.raises(ValueError):
        rog.rog_reduce([a, torch.zeros(16, dtype=torch.bfloat16, device=gpu)])
    with pytest.raises(ValueError):
        rog.rog_reduce([a, torch.zeros(15, dtype=torch.float32, device=gpu)])
    with pytest.raises(ValueError):
        rog.rog_reduce([torch.zeros(16, dtype=torch.int32, device=gpu)])
    with pytest.raises(ValueError):
        rog.rog_reduce([a.half(), a])                                        # mixed dtypes
    with pytest.raises(ValueError):
        rog.rog_reduce([a], torch.zeros(16, dtype=torch.float32))          # output on the CPU
    with pytest.raises(rog.RogArgumentError):
        rog.rog_reduce([a[:8], a[4:12]], a[4:12])                           # partial overlap


# ---------------------------------------------------------------------------
# rog_reduce_many: one launch for a batch
# ---------------------------------------------------------------------------

def _batch(seed, W, counts, dtype, offs=None, kinds=None, in_place=None):
    items = []
    for t, n in enumerate(counts):
        kind = kinds[t] if kinds else "uniform"
        payloads = wl.reduce_payloads(wl.case_seed(23, seed * 100 + t), W, n, dtype, kind)
        io = offs[t] if offs else [0] * W
        ip = in_place[t] if in_place else -1
        items.append(gc.PlacedReduce(payloads, io, t % 4, dtype, gpu_device(), in_place=ip))
    return gc.PlacedReduceBatch(items)


def gpu_device():
    return torch.device("cuda:0")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("W", [1, 3, 8])
def test_batched_sums_mixed_sizes(gpu, dtype, W):
    counts = [0, 1, 7, 513, 4096, 0, 70_001, 262_147, 9]
    offs = [[(t + r) % 4 for r in range(W)] for t in range(len(counts))]
    kinds = ["bits" if t % 3 == 0 else "uniform" for t in range(len(counts))]
    _batch(W, W, counts, dtype, offs, kinds).run("batched sums W=%d %s" % (W, dtype))


def test_batched_sums_maximum_batch(gpu):
    n = rog.rog_max_batch()
    W = rog.rog_max_batch_pointers() // n
    rng = np.random.default_rng(31)
    counts = [int(rng.integers(1, 20_000)) for _ in range(n)]
    _batch(40, W, counts, "bf16").run("batched sums max n=%d W=%d" % (n, W))


def test_batched_sums_in_place(gpu):
    counts = [1000, 33_333, 5]
    _batch(41, 4, counts, "f32", in_place=[0, 3, 1]).run("batched sums in place")


def test_batched_sums_large(gpu):
    """Sixteen bf16 tensors of the batched gather's shapes (rows up to 3000 x
    cols in {128, 1024, 8192}), W = 4, summed in one launch."""
    case = wl.config5(0, max_rows=3000)
    counts = [x.rows * x.cols for x in case.tensors]
    offs = [[(x.in_off // 2) % 4] * case.W for x in case.tensors]
    b = _batch(42, case.W, counts, "bf16", offs)
    b.run("batched sums, config-5 shapes")


def test_batched_sums_sharing_sources(gpu):
    """Two tensors summing the same source buffers into separate outputs, and
    an empty tensor whose output pointer lies inside another's output."""
    W, n = 3, 50_000
    payloads = wl.reduce_payloads(wl.case_seed(24, 0), W, n, "f32")
    a = gc.PlacedReduce(payloads, [0, 1, 2], 0, "f32", gpu)
    b = gc.PlacedReduce(payloads, [0, 0, 0], 3, "f32", gpu)
    srcs = a.srcs
    empty_out = a.out[10:10]
    outs = rog.rog_reduce_many([srcs, srcs, [s[:0] for s in srcs]], [a.out, b.out, empty_out])
    assert outs[0] is a.out and outs[1] is b.out
    a.check("shared sources, tensor 0")
    b.check("shared sources, tensor 1")


_STREAMED = {}


def _streamed_payloads(dtype, n):
    if dtype not in _STREAMED:
        _STREAMED.clear()           # one element type's 384 MiB at a time
        _STREAMED[dtype] = wl.reduce_payloads(606, 8, n, dtype, "bits" if dtype == "f16" else "uniform")
    return _STREAMED[dtype]


@pytest.mark.parametrize("offs", [((0,) * 8, 0), ((1,) * 8, 0), ((0,) * 8, 1), ((2,) * 8, 0), ((3,) * 8, 5),
                                  (tuple(range(8)), 3)], ids=lambda o: "in%s_out%d" % (o[0][:2], o[1]))
@pytest.mark.parametrize("dtype,n", [("bf16", 24 << 20), ("f32", 12 << 20), ("f16", 24 << 20)])
def test_streamed_sums_take_the_granule_form(gpu, dtype, n, offs):
    """Sums over 384 MiB of sources stream their loads and read every source as
    aligned granules shared between lanes, at any element offset: every
    element against the oracle."""
    in_offs, out_off = offs
    placed = gc.PlacedReduce(_streamed_payloads(dtype, n), in_offs, out_off, dtype, gpu)
    plan = rog.rog_reduce_plan(placed.srcs, placed.out)
    assert plan["path"] == "multi_wg" and plan["nt_loads"] and plan["shifted_loads"]
    gc.run_reduce_all_paths(placed, "streamed %s in=%s out=%d" % (dtype, in_offs, out_off),
                            paths=(rog.ROG_PATH_AUTO,))


@pytest.mark.parametrize("which,offs", [(3, ((1, 0, 3, 2, 5, 4, 7, 6), None)), (0, ((2,) * 8, None))],
                         ids=["srcs3_mixed", "srcs0_in2"])
def test_streamed_sum_in_place(gpu, which, offs):
    """An in-place sum (out is srcs[which]) over 384 MiB of sources, which takes
    the granule form: every element against the oracle, and the in-place
    buffer's own guards and every other source unchanged."""
    in_offs = offs[0]
    placed = gc.PlacedReduce(_streamed_payloads("bf16", 24 << 20), in_offs, 0, "bf16", gpu, in_place=which)
    plan = rog.rog_reduce_plan(placed.srcs, placed.out)
    assert plan["path"] == "multi_wg" and plan["nt_loads"] and plan["shifted_loads"]
    gc.run_reduce_all_paths(placed, "streamed in place srcs[%d]" % which, paths=(rog.ROG_PATH_AUTO,))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_streamed_batch_with_small_tensors(gpu, dtype):
    """A batch of sums over 128 MiB or more of sources takes the
    granule form for every tensor, down to single elements, bodies shorter
    than one wave and empty tensors: one 100 MiB-per-source tensor (W = 4)
    beside small ones at element offsets."""
    big = (100 << 20) // wl.REDUCE_ESIZE[dtype]
    counts = [big, 0, 1, 7, 127, 129, 520, 2049, 33_333, 0, 262_147]
    offs = [[(t + r) % 5 for r in range(4)] for t in range(len(counts))]
    b = _batch(43, 4, counts, dtype, offs)
    b.run("streamed batch of sums %s" % dtype)


def test_streamed_sum_of_random_bit_patterns(gpu):
    """The granule form on bf16 random bit patterns (NaNs, infinities,
    subnormals) at element offsets: 8 x 24 Mi elements, every element against
    the oracle (NaNs compared by class)."""
    payloads = wl.reduce_payloads(607, 8, 24 << 20, "bf16", "bits")
    placed = gc.PlacedReduce(payloads, (1, 0, 3, 2, 5, 4, 7, 6), 1, "bf16", gpu)
    plan = rog.rog_reduce_plan(placed.srcs, placed.out)
    assert plan["nt_loads"] and plan["shifted_loads"]
    gc.run_reduce_all_paths(placed, "streamed bf16 bit patterns", paths=(rog.ROG_PATH_AUTO,))


@pytest.mark.parametrize("W,n,dtype", [(12, 16 << 20, "bf16"), (64, 3 << 20, "f16"), (9, 11 << 20, "f32")])
def test_streamed_sums_over_several_source_groups(gpu, W, n, dtype):
    """The granule form with more sources than one group of loads in flight
    (8): W = 12, 64 and 9 over 384 MiB or more of sources, each source at its
    own element offset; every element against the oracle."""
    payloads = wl.reduce_payloads(608 + W, W, n, dtype)
    placed = gc.PlacedReduce(payloads, [r % 7 for r in range(W)], 2, dtype, gpu)
    plan = rog.rog_reduce_plan(placed.srcs, placed.out)
    assert plan["nt_loads"] and plan["shifted_loads"]
    gc.run_reduce_all_paths(placed, "streamed W=%d %s" % (W, dtype), paths=(rog.ROG_PATH_AUTO,))


@pytest.mark.parametrize("W,n,offs,nt,granule", [
    (4, 16 << 20, (1, 0), True, True), (4, (16 << 20) - 8, (1, 0), False, False),
    (3, 22_369_622, (0, 1), True, True), (2, 32 << 20, (1, 0), True, True),
    (2, (32 << 20) - 8, (1, 0), False, False), (2, 96 << 20, (0, 1), True, True)],
    ids=["4x32MiB", "4x32MiB-16B", "3x128MiB+4B", "2x64MiB", "2x64MiB-16B", "2x192MiB"])
def test_sums_around_the_streaming_bound(gpu, W, n, offs, nt, granule):
    """A sum streams its loads from 128 MiB of sources and then reads shared
    granules, two, four or eight sources at a time by W: on both sides of the
    bound, at element offsets, every element against the oracle."""
    payloads = wl.reduce_payloads(640 + W, W, n, "bf16")
    in_off, out_off = offs
    placed = gc.PlacedReduce(payloads, [in_off] * W, out_off, "bf16", gpu)
    plan = rog.rog_reduce_plan(placed.srcs, placed.out)
    assert plan["path"] == "multi_wg" and plan["nt_loads"] is nt and plan["shifted_loads"] is granule
    gc.run_reduce_all_paths(placed, "sum W=%d n=%d" % (W, n), paths=(rog.ROG_PATH_AUTO,))


def test_streamed_batch_of_sums_from_128_MiB(gpu):
    """A batch of sums streams from 128 MiB of sources, as a single sum does: 16
    tensors of 1.5 Mi bf16 elements (192 MiB of sources) at element offsets,
    every element against the oracle."""
    counts = [3 << 19] * 16
    offs = [[(t + r) % 3 for r in range(4)] for t in range(16)]
    _batch(47, 4, counts, "bf16", offs).run("batch of sums, 192 MiB of sources")


def test_streamed_batch_of_sums_with_two_sources(gpu):
    """A streamed batch of sums with 2 sources (granules two sources at a
    time): 16 tensors of 4 Mi bf16 elements (256 MiB of sources) at element
    offsets, every element against the oracle."""
    counts = [4 << 20] * 16
    offs = [[(t + r) % 3 for r in range(2)] for t in range(16)]
    _batch(48, 2, counts, "bf16", offs).run("batch of sums, W = 2, 256 MiB of sources")


@pytest.mark.parametrize("W", [2, 3])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_streamed_small_W_sums_in_every_element_type(gpu, dtype, W):
    """The granule form with two and four sources' granules in flight (W = 2
    and 3) in binary16 and binary32, just past 128 MiB of sources, sources at
    their own element offsets: every element against the oracle."""
    es = wl.REDUCE_ESIZE[dtype]
    n = (128 << 20) // (W * es) + 17
    payloads = wl.reduce_payloads(660 + W, W, n, dtype, "bits" if dtype == "f16" else "uniform")
    placed = gc.PlacedReduce(payloads, [(r * 3 + 1) % 5 for r in range(W)], 2, dtype, gpu)
    plan = rog.rog_reduce_plan(placed.srcs, placed.out)
    assert plan["path"] == "multi_wg" and plan["nt_loads"] and plan["shifted_loads"]
    gc.run_reduce_all_paths(placed, "streamed W=%d %s" % (W, dtype), paths=(rog.ROG_PATH_AUTO,))


@pytest.mark.parametrize("W", [1, 5, 6, 7])
def test_streamed_sums_with_partly_filled_groups(gpu, W):
    """Streamed bf16 sums whose sources fill their group of granules only in
    part (W = 1 of 2; W = 5, 6 and 7 of 8), just past 128 MiB of sources, at
    element offsets: every element against the oracle."""
    n = (128 << 20) // (W * 2) + 33
    payloads = wl.reduce_payloads(680 + W, W, n, "bf16")
    placed = gc.PlacedReduce(payloads, [(r * 2 + 1) % 7 for r in range(W)], 1, "bf16", gpu)
    plan = rog.rog_reduce_plan(placed.srcs, placed.out)
    assert plan["path"] == "multi_wg" and plan["nt_loads"] and plan["shifted_loads"]
    gc.run_reduce_all_paths(placed, "streamed W=%d bf16" % W, paths=(rog.ROG_PATH_AUTO,))


@pytest.mark.parametrize("W,in_offs,tail", [
    (4, (0, 64, 8, 200), 48),
    (6, (0, 0, 64, 0, 128, 448), 400),
    (8, (0, 64, 128, 8, 0, 72, 200, 16), 48),
    (8, (0, 1, 64, 3, 0, 8, 5, 192), 400)],
    ids=["W4_aligned", "W6_aligned", "W8_aligned", "W8_mixed"])
def test_streamed_aligned_sums_with_a_short_last_chunk(gpu, W, in_offs, tail):
    """Streamed sums (just past 128 MiB of sources) whose aligned sources sit
    on assorted 128-byte line places, the body ending `tail` bytes into its
    last 1 KiB chunk: from W = 4 the last lane of each wave reads an aligned
    source's granule of the next chunk at a line chosen by rank, inside the
    body only; the mixed case has misaligned sources beside aligned ones.
    Source 0 sits 64 bytes past a line (the guard), so the body starts 64
    bytes in.  Every element against the oracle."""
    n = ((128 << 20) // (2 * W) // 512 + 1) * 512 + (64 + tail) // 2
    assert (2 * n - 64) % 1024 == tail and wl.GUARD == 64
    payloads = wl.reduce_payloads(700 + W + sum(in_offs), W, n, "bf16")
    placed = gc.PlacedReduce(payloads, in_offs, 0, "bf16", gpu)
    plan = rog.rog_reduce_plan(placed.srcs, placed.out)
    assert plan["path"] == "multi_wg" and plan["nt_loads"] and plan["shifted_loads"]
    gc.run_reduce_all_paths(placed, "streamed aligned W=%d offs=%s" % (W, in_offs), paths=(rog.ROG_PATH_AUTO,))


def test_largest_sum(gpu):
    """A sum at the top of the size range: W = 2 bf16 sources of 2^35 - 64
    elements (an output of 2^36 - 128 bytes), the sources one element off the
    output, so streamed loads and the granule form.  Checked through
    properties that hold at any size: sampled windows at both ends and in the
    middle equal a float32 sum in rank order rounded once to bf16, and the
    filled stretches between them hold the exact sum of the fill values."""
    W = 2
    n = (1 << 35) - 64
    free, _ = torch.cuda.mem_get_info(gpu)
    need = (W + 1) * 2 * n
    if free < need + (8 << 30):
        pytest.skip("needs %d GiB of free device memory" % ((need >> 30) + 8))
    fills = (1.5, 0.25)                      # 1.75: exact in bf16
    bufs, srcs = [], []
    for r in range(W):
        t = torch.empty(n + 1, dtype=torch.bfloat16, device=gpu)
        t.fill_(fills[r])
        bufs.append(t)
        srcs.append(t[1:])
    g = torch.Generator(device=gpu)
    g.manual_seed(97)
    win = 8192
    windows = [0, n - win, n // 2 + 5]
    for r in range(W):
        for lo in windows:
            srcs[r][lo:lo + win].copy_(torch.randn(win, device=gpu, generator=g).to(torch.bfloat16))
    out = torch.empty(n, dtype=torch.bfloat16, device=gpu)
    plan = rog.rog_reduce_plan(srcs, out)
    assert plan["path"] == "multi_wg" and plan["nt_loads"] and plan["shifted_loads"]
    print("largest sum W=2 n=%d" % n, flush=True)
    rog.rog_reduce(srcs, out)
    torch.cuda.synchronize()
    for lo in windows:
        want = (srcs[0][lo:lo + win].float() + srcs[1][lo:lo + win].float()).to(torch.bfloat16)
        assert torch.equal(out[lo:lo + win].view(torch.int16).cpu(), want.view(torch.int16).cpu()), lo
    mid = out[win: win + (1 << 20)].float().cpu()
    assert torch.all(mid == 1.75)
    del out, srcs, bufs
    torch.cuda.empty_cache()
