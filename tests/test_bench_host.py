"""Host-side parts of bench.py that need no GPU: the amd-smi telemetry parser
(on the JSON shape amd-smi prints for an MI355X: one gfx clock per XCD and a
hotspot temperature) and the host CPU record."""
from __future__ import annotations

import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def _clk(v):
    return {"clk": {"value": v, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
            "max_clk": {"value": 2400, "unit": "MHz"}, "clk_locked": "DISABLED", "deep_sleep": "ENABLED"}


def _gpu(i, clocks, hot):
    clock = {"gfx_%d" % x: _clk(c) for x, c in enumerate(clocks)}
    clock["mem_0"] = _clk(1900)  # not an engine clock
    return {"gpu": i, "clock": clock,
            "temperature": {"edge": "N/A", "hotspot": {"value": hot, "unit": "C"}, "mem": {"value": 34, "unit": "C"}}}


def test_parse_one_device():
    data = {"gpu_data": [_gpu(0, [2300, 2310, 2290, 2300, 2305, 2295, 2300, 2300], 71)]}
    assert bench.GpuTelemetry.parse(data) == (2300.0, 71)


def test_parse_picks_the_busy_device_and_tolerates_na():
    idle = _gpu(0, [150] * 8, 40)
    busy = _gpu(1, [2350] * 8, 80)
    busy["temperature"]["hotspot"] = "N/A"
    assert bench.GpuTelemetry.parse({"gpu_data": [idle, busy]}) == (2350.0, None)


def test_parse_without_clocks_raises():
    try:
        bench.GpuTelemetry.parse({"gpu_data": [{"gpu": 0, "clock": {"mem_0": _clk(1900)}}]})
    except ValueError:
        return
    raise AssertionError("expected ValueError")


def test_summary_of_samples():
    t = bench.GpuTelemetry(interval_s=0.05)
    t.clocks, t.temps = [2300.0, 2340.0], [70, 75]
    s = t.summary()
    assert s["samples"] == 2 and s["gfx_clock_mhz"]["min"] == 2300.0 and s["gfx_clock_mhz"]["max"] == 2340.0
    assert s["hotspot_c_max"] == 75


def test_host_cpu_record():
    h = bench.host_cpu()
    assert h["threads_available"] >= 1
    assert h["smt"] in (True, False, None)


def test_disabled_telemetry_starts_nothing():
    t = bench.GpuTelemetry(enabled=False)
    with t:
        pass
    assert not t._thread.is_alive() and t.summary() == {"samples": 0, "skipped": "--no-telemetry"}


def test_kernel_hash_ignores_comments_not_code():
    src = 'int f(int a) { // add one\n    return a + 1; /* the\n answer */ }\nconst char *s = "x // y";\n'
    commented = '// header\n' + src.replace('// add one', '// adds one to a')
    changed = src.replace('a + 1', 'a + 2')
    literal = src.replace('"x // y"', '"x // z"')
    assert bench.strip_c_comments(src) == bench.strip_c_comments(commented)
    assert bench.strip_c_comments(src) != bench.strip_c_comments(changed)
    assert bench.strip_c_comments(src) != bench.strip_c_comments(literal)  # strings are code

