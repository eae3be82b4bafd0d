"""Host-side tooling of the measurement (CPU only): the bench's contract
checks, its rotation sizing and repeat statistics, the gating of the counter
traffic by the GEMV sources, and the rocprofv3 summaries on synthetic CSVs."""

import csv
import os
import subprocess
import sys

import pytest

import bench
from skinny_gemm_decode_amd import rocprof_summary as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("nbytes", [139_264, 33_030_144, 62_390_272, 100_663_296, 3 * 10**9])
def test_rotation_covers_two_gigabytes(nbytes):
    n = bench.rotation_count(nbytes)
    assert n >= 1
    assert n * nbytes >= 2 * 1000**3 or n == 1
    assert (n - 1) * nbytes < 2 * 1000**3


def test_summarize_spread_and_gate():
    r = bench.summarize([10.0, 10.2, 9.8, 10.0], total_ms=8.0, launches=800)
    assert r["us_per_launch"] == pytest.approx(10.0)
    assert r["spread"] == pytest.approx(0.4 / 10.0)
    assert r["spread_ok"]
    assert not bench.summarize([10.0, 11.0], 2.1, 200)["spread_ok"]
    # one repeat has no spread, and no spread claim can be made from it
    one = bench.summarize([10.0], 2.0, 200)
    assert one["spread"] is None and not one["spread_ok"]


def test_protocol_needs_warmup_repeats_and_spread():
    good = {"warm_s": 1.2, "repeats": 10, "launches_per_repeat": 200, "spread_ok": True}
    assert bench.protocol_ok(good)
    for k, v in (("warm_s", 0.3), ("repeats", 9), ("launches_per_repeat", 20), ("spread_ok", False)):
        assert not bench.protocol_ok(dict(good, **{k: v})), k


def test_timer_runs_warmup_then_exact_repeats():
    """Warm-up repeats (topped up to the requested seconds), then exactly the
    requested repeats of per_repeat launches, each between two events."""
    launched = []

    class Ev:
        n = 0

        def __init__(self, enable_timing=True):
            self.t = None

        def record(self, stream):
            self.t = float(len(launched))

        def elapsed_time(self, other):
            return (other.t - self.t) * 0.01           # 10 us per launch, in ms

    class FakeCuda:
        Event = Ev

        @staticmethod
        def current_stream():
            return type("S", (), {"cuda_stream": 0})()

        @staticmethod
        def synchronize():
            pass

    class FakeTorch:
        cuda = FakeCuda

    r = bench.Timer(FakeTorch).run(lambda i, sh: launched.append(i), 7, repeats=3, per_repeat=50, warm_repeats=2,
                                   warm_s=0.0)
    assert len(launched) == 2 * 50 + 3 * 50
    assert launched[:5] == [0, 1, 2, 3, 4] and launched[100] == 100 % 7
    assert r["repeats"] == 3 and r["launches_per_repeat"] == 50 and r["warm_repeats"] == 2
    assert r["us_per_launch"] == pytest.approx(10.0) and r["spread"] == pytest.approx(0.0)


def test_counter_traffic_is_gated_by_the_gemv_sources(tmp_path, monkeypatch):
    good = tmp_path / "good.md"
    good.write_text(f"x\n    traffic_bytes_per_launch: 123456\n    gemv_source_sha256: {rs.gemv_source_hash()}\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(good))
    assert bench.counter_traffic() == 123456
    stale = tmp_path / "stale.md"
    stale.write_text("    traffic_bytes_per_launch: 123456\n    gemv_source_sha256: " + "0" * 64 + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(stale))
    assert bench.counter_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "missing.md"))
    assert bench.counter_traffic() is None


def _counter_csv(path, rows):
    path.mkdir(parents=True, exist_ok=True)
    with open(path / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, c, v) in enumerate(rows):
            w.writerow([i, k, c, v])


def test_traffic_md_scales_by_the_copy(tmp_path):
    gemv = "void skg::gemv_kernel<0, 1, 2, 1, false, 8, 0, 8>(skg::GemvArgs)"
    read = "skg::stream_read_kernel(uint4 const*, long, unsigned int, unsigned int*)"
    copy = "__amd_rocclr_copyBuffer"
    mib256 = (1 << 28) / 1024.0
    # FETCH reads half the bytes (x2 scale), WRITE exact; a smaller copy must not set the scale
    _counter_csv(tmp_path / "f", [(gemv, "FETCH_SIZE", 49000.0), (gemv, "FETCH_SIZE", 49400.0),
                                  (read, "FETCH_SIZE", 49100.0), (copy, "FETCH_SIZE", 10.0),
                                  (copy, "FETCH_SIZE", mib256 / 2)])
    _counter_csv(tmp_path / "w", [(gemv, "WRITE_SIZE", 192.0), (copy, "WRITE_SIZE", 5.0),
                                  (copy, "WRITE_SIZE", mib256)])
    md = rs.traffic_md(str(tmp_path / "f"), str(tmp_path / "w"))
    expect = int(round((49200.0 * 2.0 + 192.0) * 1024))
    assert f"traffic_bytes_per_launch: {expect}" in md
    assert "FETCH_SIZE is scaled by 2.0000 and WRITE_SIZE by 1.0000" in md
    assert f"gemv_source_sha256: {rs.gemv_source_hash()}" in md


def test_trace_and_counter_tables_keep_only_library_kernels(tmp_path):
    d = tmp_path / "t"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["void skg::gemv_kernel<0, 1>(skg::GemvArgs)", 10, 157000, 15700, 90, 15000, 16500, 1])
        w.writerow(["at::native::elementwise_kernel<...>(...)", 5, 5000, 1000, 10, 900, 1100, 1])
    md = rs.trace_md(str(d), "T", "cmd --x")
    assert "| `void skg::gemv_kernel<0, 1>` | 10 | 15.700 | 15.000 | 16.500 |" in md
    assert "elementwise" not in md and "    cmd --x" in md
    _counter_csv(tmp_path / "c1", [("skg::quantize_q8_1_kernel(float const*)", "SQ_WAVES", 4.0),
                                   ("skg::quantize_q8_1_kernel(float const*)", "SQ_WAVES", 6.0),
                                   ("at::native::foo", "SQ_WAVES", 1.0)])
    _counter_csv(tmp_path / "c2", [("skg::quantize_q8_1_kernel(float const*)", "SQ_BUSY_CYCLES", 100.0)])
    md = rs.counters_md("C", "a ;; b", [str(tmp_path / "c1"), str(tmp_path / "c2")])
    assert "| kernel | dispatches | SQ_BUSY_CYCLES | SQ_WAVES |" in md
    assert "| `skg::quantize_q8_1_kernel` | 2 | 100 | 5 |" in md
    assert "    a\n    b" in md and "foo" not in md


def test_telemetry_reads_the_device_torch_uses(tmp_path):
    """Clock levels (the starred pp_dpm line), hwmon temperatures and power of
    the card whose PCI bus torch reports; other cards are ignored."""
    for card, slot, sclk in (("card0", "0000:11:00.0", "2100"), ("card1", "0000:75:00.0", "2400")):
        d = tmp_path / card / "device"
        (d / "hwmon" / "hwmon3").mkdir(parents=True)
        (d / "uevent").write_text(f"DRIVER=amdgpu\nPCI_SLOT_NAME={slot}\n")
        (d / "pp_dpm_sclk").write_text(f"0: 500Mhz\n1: {sclk}Mhz *\n")
        (d / "pp_dpm_mclk").write_text("0: 2000Mhz *\n")
        (d / "hwmon" / "hwmon3" / "temp2_input").write_text("61000\n")
        (d / "hwmon" / "hwmon3" / "temp3_input").write_text("48000\n")
        (d / "hwmon" / "hwmon3" / "power1_input").write_text("812000000\n")

    class FakeTorch:
        class cuda:
            @staticmethod
            def get_device_properties(i):
                return type("P", (), {"pci_bus_id": 0x75})()

    t = bench.Telemetry(FakeTorch, root=str(tmp_path))
    r = t.read()
    assert r == {"sclk_mhz": 2400.0, "mclk_mhz": 2000.0, "t_junction_c": 61.0, "t_mem_c": 48.0, "power_w": 812.0}
    assert bench.Telemetry.summary([r, None, dict(r, sclk_mhz=2300.0)])["sclk_mhz"] == [2300.0, 2400.0]
    assert bench.Telemetry(FakeTorch, root=str(tmp_path / "none")).read() is None


def test_abba_order_and_ratio():
    """Legs run A1 B1 B2 A2 per cycle and the ratio is the mean of the cycle
    ratios; a linear drift across a cycle cancels."""
    calls = []

    class FakeTimer:
        t = 0.0

        def run(self, f, n_rot, repeats=10, **kw):
            calls.append(f.__name__)
            FakeTimer.t += 1.0                       # drift: every leg 1 us slower than the last
            base = 10.0 if f.__name__ == "a" else 12.0
            return {"us_per_launch": base + FakeTimer.t}

    def a(i, sh):
        pass

    def b(i, sh):
        pass

    r = bench.compare_abba(FakeTimer(), a, b, 4, 100, cycles=2)
    assert calls == ["a", "b", "b", "a"] * 2
    # cycle 1: A legs 11, 14 -> 12.5; B legs 14, 15 -> 14.5 (drift cancels in the means' centres)
    assert r["cycles"][0]["b_over_a"] == pytest.approx(14.5 / 12.5)
    assert r["b_over_a"] == pytest.approx((14.5 / 12.5 + 18.5 / 16.5) / 2)


def test_sweep_takes_k4096_restates_the_shape_rules():
    """The bench's sweep arm times only variants that accept K = 4096: the
    LDS ring needs waves x kw = 128 blocks, the register-fed matrix-core
    kernel kw | 128 <= waves x kw, the LDS-staged K split an equal number of
    chunks per K class."""
    import bench
    v = dict(fmt=2, M=8, epi=0, ro=16, j=1, x_lds=3, waves=8, kw=16, depth=2)
    assert bench.takes_k4096(v)
    assert not bench.takes_k4096(dict(v, kw=8))
    assert bench.takes_k4096(dict(v, x_lds=2, waves=16, kw=8))
    assert not bench.takes_k4096(dict(v, x_lds=2, waves=4, kw=8))
    assert bench.takes_k4096(dict(v, x_lds=1, j=1, kw=2, ro=4, waves=4))      # 2 chunks of 64 units
    assert not bench.takes_k4096(dict(v, x_lds=1, j=2, kw=2, ro=4, waves=4))  # 1 chunk of 128
    assert bench.takes_k4096(dict(v, x_lds=0, j=2, kw=1, ro=4, waves=4))
