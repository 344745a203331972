"""bench.py's arithmetic and JSON contract on the CPU, with made-up timings
(the idea of the pages' benchmark unit tests, which run the harness against a
mocked event class: RL-Align/RL-Kernel PR #491, author's replies on the
benchmark tests)."""
from __future__ import annotations

import json
import os

import pytest

import bench


def test_percentile_and_summary():
    xs = [5.0, 1.0, 3.0, 2.0, 4.0]
    assert bench.percentile(xs, 50) == 3.0
    assert bench.percentile(xs, 0) == 1.0
    assert bench.percentile(xs, 100) == 5.0
    assert bench.percentile(xs, 25) == 2.0
    assert bench.percentile([7.0], 90) == 7.0
    s = bench.summarize_ms([0.010, 0.020, 0.030])
    assert s["p50_us"] == pytest.approx(20.0)
    assert s["n"] == 3
    with pytest.raises(ValueError):
        bench.percentile([], 50)


def test_gbps_and_roofline():
    # 1 GiB moved in 0.2 ms
    one_gib = 1 << 30
    assert bench.gbps(one_gib, 0.2) == pytest.approx(one_gib / 2e-4 / 1e9)
    r = bench.roofline(one_gib, 0.2, traffic=1.07e9)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, rel=1e-3)
    assert r["traffic"] == 1070000000
    assert bench.roofline(one_gib, 0.2, traffic=None)["traffic"] is None


def test_json_line_contract():
    line = bench.build_line(value=5000.0, steps=100, warmup=10, ms_per_step=0.2,
                            config={"workload": "x"}, roof=bench.roofline(1 << 30, 0.2, None),
                            cpu={"value": 1.0, "unit": "GB/s", "cores": 1, "kind": "oracle", "sample": "s"},
                            extras={"latency": []})
    s = json.dumps(line)
    back = json.loads(s)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in back, k
    assert back["metric"] == bench.METRIC and "GB/s" in back["metric"] and "p50" in back["metric"]
    assert back["n_gpus"] == 1 and back["higher_is_better"] is True and back["vs_baseline"] is None
    assert back["config"]["workload"] == "x"
    assert "model" not in back["config"]


def test_traffic_file_is_ignored_when_kernel_sources_change(tmp_path):
    digest = bench.kernel_source_digest()
    p = tmp_path / "t.md"
    p.write_text("kernel_source_sha256: %s\ntraffic_bytes_per_launch: 1.1e9\n" % digest)
    assert bench.read_traffic(str(p), digest) == pytest.approx(1.1e9)
    assert bench.read_traffic(str(p), "0" * 64) is None
    assert bench.read_traffic(str(tmp_path / "missing.md"), digest) is None
    p.write_text("nothing here\n")
    assert bench.read_traffic(str(p), digest) is None


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_bad_step_counts_are_refused():
    assert bench.main(["--steps", "0"]) == 2
    assert bench.main(["--warmup", "-1"]) == 2


class FakeEvent:
    """Stands in for torch.cuda.Event: times come from a scripted clock."""
    clock = [0.0]

    def __init__(self, enable_timing=True):
        self.t = None

    def record(self):
        self.t = FakeEvent.clock[0]

    def elapsed_time(self, other):
        return other.t - self.t


class FakeCuda:
    Event = FakeEvent

    @staticmethod
    def synchronize():
        pass


class FakeTorch:
    cuda = FakeCuda


def test_time_region_spans_only_the_timed_calls():
    calls = []

    def fn():
        calls.append(1)
        FakeEvent.clock[0] += 3.0 if len(calls) <= 2 else 0.5
    FakeEvent.clock[0] = 0.0
    assert bench.time_region(FakeTorch, fn, steps=4, warmup=2) == pytest.approx(2.0)
    assert len(calls) == 6


def test_time_calls_attributes_each_interval_to_its_call():
    durations = [0.5, 0.25, 1.0, 0.125]
    calls = []

    def fn():
        i = len(calls)
        calls.append(i)
        FakeEvent.clock[0] += durations[i - 2] if i >= 2 else 7.0   # 2 warmups
    FakeEvent.clock[0] = 0.0
    per_call, region = bench.time_calls(FakeTorch, fn, steps=4, warmup=2)
    assert per_call == durations
    assert region == pytest.approx(sum(durations))
    assert len(calls) == 6


def test_source_digest_ignores_comments_but_not_code(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("// header\nint f(int x) {  /* twice */ return 2 * x; }  // tail\n")
    d0 = bench.kernel_source_digest([str(a)])
    a.write_text("// a new header\n\nint f(int x) {\n    /* doubled */\n    return 2 * x;\n}\n")
    assert bench.kernel_source_digest([str(a)]) == d0
    a.write_text("int f(int x) { return 3 * x; }\n")
    assert bench.kernel_source_digest([str(a)]) != d0


def test_hip_attribute_numbers_match_the_header(tmp_path):
    """The bench reads the memory bus width and clock with hipDeviceGetAttribute;
    its enum numbers must be the ones the installed HIP header defines."""
    import shutil
    import subprocess
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h") or not shutil.which("gcc"):
        pytest.skip("no HIP header or gcc")
    src = tmp_path / "attr.c"
    src.write_text('#include <hip/hip_runtime_api.h>\n#include <stdio.h>\n'
                   'int main(void) { printf("%d %d", (int)hipDeviceAttributeMemoryBusWidth, '
                   '(int)hipDeviceAttributeMemoryClockRate); return 0; }\n')
    exe = tmp_path / "attr"
    subprocess.check_call(["gcc", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", str(src), "-o", str(exe)])
    bus, clock = map(int, subprocess.check_output([str(exe)]).split())
    assert (bench.HIP_ATTR_MEMORY_BUS_WIDTH, bench.HIP_ATTR_MEMORY_CLOCK_RATE) == (bus, clock)


def test_host_cpu_reports_model_and_cores():
    h = bench.host_cpu()
    assert h["cores_available"] >= 1


def test_native_latency_harness_builds():
    """bench_native.c (small-gather latency timed from C) compiles against the
    installed header and librog.so; bench.py runs the binary on the GPU."""
    import shutil
    if not shutil.which("gcc") or not os.path.exists(os.path.join(bench.ROOT, "deterministic_collective_movement_amd",
                                                                  "librog.so")):
        pytest.skip("no gcc or librog.so not built")
    path = bench.build_native()
    assert os.access(path, os.X_OK)


def test_slices_cover_the_range_once():
    for n, parts in [(10, 3), (7, 7), (5, 9), (1 << 20, 64), (1, 1)]:
        pieces = bench.slices(n, parts)
        assert pieces[0][0] == 0 and pieces[-1][1] == n
        assert all(a[1] == b[0] for a, b in zip(pieces, pieces[1:]))
        assert all(hi > lo for lo, hi in pieces)
        assert len(pieces) == min(parts, n)


def test_cpu_baselines_report_cores_and_the_single_core_figure():
    """Both oracle legs on a small stand-in case: the line carries the
    many-core figure with its thread count, the single-core one beside it,
    and the many-core results equal the single-call ones."""
    import numpy as np
    from deterministic_collective_movement_amd import workloads as wl
    from oracle import oracle

    class Case:
        W, S = 3, 100_003
    payloads = [wl.random_bytes(5, r, Case.S) for r in range(Case.W)]
    cpu = bench.cpu_baseline(Case, payloads, 0.05, threads=4)
    assert cpu["kind"] == "oracle" and cpu["cores"] == 4 and cpu["unit"] == "GB/s" and cpu["value"] > 0
    assert cpu["single_core"]["cores"] == 1 and cpu["single_core"]["value"] > 0
    assert "cpu_model" in cpu and cpu["cores_available"] >= 1
    rp = wl.reduce_payloads(6, 8, 5000, "bf16")
    want = np.empty(5000, np.uint16)
    oracle.reduce_c(rp, want, "bf16")
    red = bench.reduce_cpu_baseline(rp, want, 0.05, sample=5000, threads=3)
    assert red["cores"] == 3 and red["single_core"]["cores"] == 1
    with pytest.raises(AssertionError):
        bad = want.copy()
        bad[7] ^= 1
        bench.reduce_cpu_baseline(rp, bad, 0.01, sample=5000, threads=2)


def test_latency_legs_time_a_fixed_hundred_calls():
    import inspect
    for fn in (bench.latency_sweep, bench.reduce_latency, bench.launch_floor):
        params = inspect.signature(fn).parameters
        assert params["steps"].default == bench.LATENCY_CALLS == 100


def test_one_launch_bound_recovers_the_stream_rate_and_the_floor():
    """Gathers whose cold time is exactly floor + bytes / rate: the bound finds
    that rate from the 128 and 512 MiB rows and puts every row at its own time;
    a row slower than the bound stays above it."""
    import bench
    rate, floor = 6800.0, 1.65          # GB/s, µs
    rows = []
    for W in (2, 8):
        for mib in (64, 128, 256, 512):
            moved = 2 * mib * (1 << 20)
            t = floor + moved / (rate * 1e3) + (0.9 if mib == 64 else 0.0)   # 64 MiB: 0.9 µs of ramp
            rows.append({"W": W, "out_MiB": mib, "cold_us_per_gather": t,
                         "cold_pct_of_peak": 100 * moved / (t * 1e3) / bench.PEAK_HBM_GBPS})
    b = bench.one_launch_bound(rows, floor)
    assert b["floor_us_per_launch"] == 1.65
    assert set(b["cold_stream_GBps"]) == {"2", "8"}
    assert all(abs(v - rate) < 0.2 for v in b["cold_stream_GBps"].values())
    assert len(b["rows"]) == 8
    for r in b["rows"]:
        moved = 2 * r["out_MiB"] * (1 << 20)
        assert abs(r["bound_us"] - (floor + moved / (rate * 1e3))) < 0.01
        if r["out_MiB"] == 64:
            assert r["bound_pct_of_peak"] > r["cold_pct_of_peak"]
        else:
            assert abs(r["bound_pct_of_peak"] - r["cold_pct_of_peak"]) < 0.1
    # rows without both reference sizes give no rate
    assert bench.one_launch_bound([x for x in rows if x["out_MiB"] != 512], floor)["rows"] == []
