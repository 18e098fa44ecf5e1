"""Benchmark: exhaustive search of the dense n=48 int32 QUBO on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C4] [--no-cpu]

One step is one full qubo_search call on the 2^48-state workload (fold, plan,
cache builders, Gray-walk search, reduction, result download) with Q already
resident in HBM.  Prints one JSON line with states/s, the search kernel's
roofline position (int32 VALU) and the CPU oracle timed on a bounded slice of
the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "states/sec (×10^12) on dense n=48 int32 QUBO, 1 MI355X; % of int32 VALU peak"

# MI355X int32 vector peak for two-operand adds: 256 CUs x 4 SIMDs x 32 lanes per
# clock x 2.4 GHz = 78.6e12 lane-ops/s, the lane rate behind the 157.3 TFLOP/s
# fp32 vector figure (an FMA counts 2 flops).  gfx950 retires a wave64 VOP2
# integer add in 2 cycles (measured: 7.2e13 lane-ops/s with an inline-constant
# operand, 6.7e13 with two VGPRs); three-VGPR VOP3 ops such as v_min3_i32 and
# ops with an SGPR operand take 4 cycles.
CUS, LANES_PER_CU_CLOCK, CLOCK_HZ = 256, 128, 2.4e9
INT32_VALU_PEAK = CUS * LANES_PER_CU_CLOCK * CLOCK_HZ  # 7.86e13 lane-ops/s

# Algorithmic work per state: one int32 add (eq. 9 of the paper: the suffix
# vector moves by one row per Gray step, a single integer operation per state).
# The strict kernel (Algorithm 2 as printed) also compares every state with the
# threshold: two ops per state, reported for that kernel.
OPS_PER_STATE = 1
OPS_PER_STATE_STRICT = 2

PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "gray_search_gated_n48_counters.json")
# What the counted launch is built from: the kernel source and header, the planner
# (split, segments, LDS rows) and the host run that sizes the grid, and the
# compiler flags.
KERNEL_INPUTS = [os.path.join(ROOT, "ising_ground_state_amd", "csrc", name)
                 for name in ("kernels.hip", "kernels.h", "walk.h", "dpp.h", "plan.cpp", "plan.h", "run_int.hip")]


_C_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"', re.S)


def strip_c_comments(text: str) -> str:
    """C/C++ source without its comments (string literals kept as they are),
    every run of white space collapsed to one blank."""
    code = _C_TOKENS.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
    return re.sub(r"\s+", " ", code).strip()


def kernel_source_hash() -> str:
    """Identifies the counted search launch: the kernel, planner and host-run
    sources without comments, and the compiler flags (counters taken before a
    comment edit stay valid)."""
    from ising_ground_state_amd import build as libbuild
    h = hashlib.sha256()
    for path in KERNEL_INPUTS:
        with open(path, encoding="utf-8") as f:
            h.update(strip_c_comments(f.read()).encode())
    h.update(repr(libbuild.FLAGS).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per search launch from committed rocprofv3 counter runs, or None
    when they are missing or the kernel source changed since they were taken."""
    try:
        with open(PROFILE_COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def covers(t, A, B):
    """A search's timing shows every 32-step body of 2^A Gray steps walked once
    per column group of 64 x (its columns per lane) columns."""
    group = 64 * t["cols_per_lane"]
    cols_padded = -(-(1 << B) // group) * group
    return group > 0 and t["bodies"] * 32 * group == (1 << A) * cols_padded


CPU_SAMPLE_FREE_BITS = 36
CPU_SAMPLE_SEED = 4242


def cpu_baseline(cfg):
    """The CPU oracle (tier B, Gray walk) as it stands, on every hardware thread
    this process may run on, over a seeded sub-cube of the same workload: the
    first n - 36 variables fixed to a value drawn with seed 4242, 2^36 states.
    Tier A (every state from the definition) on the whole n = 24 workload."""
    import oracle
    import qubo_instances as qi

    n = cfg["n"]
    threads = len(os.sched_getaffinity(0))
    free = CPU_SAMPLE_FREE_BITS
    k = n - free
    rng = qi.SplitMix64(CPU_SAMPLE_SEED)
    top = rng.uniform_int(0, (1 << k) - 1)
    t0 = time.perf_counter()
    r = oracle.search_gray(cfg["Q"], k=k, top=top, threads=threads)
    dt = time.perf_counter() - t0
    states = 1 << free
    c1 = qi.make_config("C1")
    t1 = time.perf_counter()
    oracle.search_direct(c1["Q"], threads=threads)
    dt_a = time.perf_counter() - t1
    return {"value": states / dt / 1e12, "unit": "1e12 states/s", "cores": threads, "kind": "oracle",
            "host": host_cpu(),
            "sample": "tier-B Gray walk over the sub-cube of 2^%d states with the first %d variables "
                      "fixed to %d (seed %d); %.2f s wall on %d threads" % (free, k, top, CPU_SAMPLE_SEED, dt,
                                                                            threads),
            "states": states, "seconds": dt, "subcube_result": list(r.triple()),
            "tier_a_c1": {"value": (1 << c1["n"]) / dt_a / 1e12, "unit": "1e12 states/s", "seconds": dt_a,
                          "sample": "tier A (direct O(n^2) per state), all 2^%d states of C1" % c1["n"]}}


def host_cpu():
    """The host's CPU model, its logical CPUs, the threads this process may run
    on, and SMT."""
    model, siblings, cores = None, None, None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name" and model is None:
                    model = val
                elif key == "siblings" and siblings is None:
                    siblings = int(val)
                elif key == "cpu cores" and cores is None:
                    cores = int(val)
    except OSError:
        pass
    smt = None if siblings is None or cores is None else siblings > cores
    return {"model": model, "nproc": os.cpu_count(), "threads_available": len(os.sched_getaffinity(0)),
            "smt": smt}


class GpuTelemetry:
    """Samples the engine clock of every XCD and the hotspot temperature with
    amd-smi, in a thread of its own, while the timed steps run.  A missing or
    failing amd-smi only leaves the record empty."""

    def __init__(self, interval_s: float = 2.0, enabled: bool = True):
        self.interval_s = interval_s
        self.enabled = enabled
        self.clocks, self.temps, self.errors = [], [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def parse(data):
        """(mean gfx clock over the XCDs in MHz, hotspot temperature in C or None)
        of the busiest device in the JSON of `amd-smi metric --clock --temperature`."""
        gpus = data["gpu_data"] if isinstance(data, dict) else data
        best = None
        for g in gpus:
            clk = [v["clk"]["value"] for k, v in g.get("clock", {}).items()
                   if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
                   and isinstance(v["clk"].get("value"), (int, float))]
            if clk and (best is None or sum(clk) / len(clk) > best[0]):
                hot = g.get("temperature", {}).get("hotspot")
                temp = hot.get("value") if isinstance(hot, dict) else None
                best = (sum(clk) / len(clk), temp if isinstance(temp, (int, float)) else None)
        if best is None:
            raise ValueError("no gfx clock in amd-smi output")
        return best

    def _sample(self):
        out = subprocess.run(["amd-smi", "metric", "--clock", "--temperature", "--json"],
                             capture_output=True, text=True, timeout=30)
        clk, temp = self.parse(json.loads(out.stdout))
        self.clocks.append(clk)
        if temp is not None:
            self.temps.append(temp)

    def _run(self):
        while not self._stop.is_set():
            try:
                self._sample()
            except Exception as e:  # telemetry is context: never fail the benchmark for it
                self.errors.append("%s: %s" % (type(e).__name__, e))
                if len(self.errors) >= 3:
                    return
            self._stop.wait(self.interval_s)

    def __enter__(self):
        if self.enabled:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.enabled:
            self._thread.join(timeout=60)

    def summary(self):
        if not self.enabled:
            return {"samples": 0, "skipped": "--no-telemetry"}
        rec = {"source": "amd-smi metric --clock --temperature, every %g s during the timed steps"
                         % self.interval_s, "samples": len(self.clocks)}
        if self.clocks:
            rec["gfx_clock_mhz"] = {"min": min(self.clocks), "mean": round(sum(self.clocks) / len(self.clocks), 1),
                                    "max": max(self.clocks), "note": "mean over the XCDs of one sample"}
        if self.temps:
            rec["hotspot_c_max"] = max(self.temps)
        if self.errors:
            rec["errors"] = self.errors[:3]
        return rec


def copy_calibration(mib: int):
    """A plain copy kernel of known size: reads and writes mib MiB once each."""
    import torch
    src = torch.ones(mib << 18, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": mib << 20, "copy_calibration_bytes_written": mib << 20}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="C4")
    ap.add_argument("--prefix-bits", type=int, default=None)
    ap.add_argument("--cache-bits", type=int, default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-telemetry", action="store_true",
                    help="no amd-smi sampling (for runs under a profiler, whose preloaded library has "
                         "initialised the GPU before this program starts: a child process would be an exec "
                         "after GPU initialisation)")
    ap.add_argument("--strict", action="store_true",
                    help="time the strict kernel (minimum after every prefix) instead of the default")
    ap.add_argument("--no-strict-leg", action="store_true",
                    help="skip the extra strict-kernel step reported beside the default mode")
    ap.add_argument("--no-f64-leg", action="store_true",
                    help="skip the extra step of the real-valued (binary64) search of C4f")
    ap.add_argument("--no-spectrum-leg", action="store_true",
                    help="skip the extra step of the 64-lowest-states search reported beside the minimum")
    ap.add_argument("--no-config-legs", action="store_true",
                    help="skip the one-search legs of the other workloads (C1, C2, C2p, C3, C5)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (for scaling HBM counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="only time one search per split of the grid below on --config (one JSON line "
                         "per point, then a summary line); every point must give the same result")
    ap.add_argument("--sweep-prefix", default="24,26,28,30,32", help="prefix_bits values of the sweep")
    ap.add_argument("--sweep-cache", default="8,10,12,13,14,16,18", help="cache_bits values of the sweep")
    ap.add_argument("--sizes", default=None, metavar="LO-HI",
                    help="instead of the benchmark: one whole-space search per size n in LO..HI (the "
                         "analogue of P1's Table IV), one JSON line per size")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the work units of one search are independent and would be split across GPUs, "
              "with one 24-byte result per GPU combined at the end)", file=sys.stderr)
        sys.exit(2)

    import torch
    import ising_ground_state_amd as q
    import qubo_instances as qi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    q.load()
    if args.sizes:
        lo, hi = (int(v) for v in args.sizes.split("-"))
        size_scan(q, lo, hi)
        return
    cfg = qi.make_config(args.config)
    n = cfg["n"]
    Qd = torch.tensor(cfg["Q"], dtype=torch.int32, device="cuda:0")
    if args.sweep:
        split_sweep(q, Qd, cfg, [int(v) for v in args.sweep_prefix.split(",")],
                    [int(v) for v in args.sweep_cache.split(",")])
        return
    plan = q.make_plan(n, args.prefix_bits, args.cache_bits)
    states = 1 << n

    for _ in range(args.warmup):
        q.search(Qd, args.prefix_bits, args.cache_bits, strict=args.strict)
        print("[bench] warmup", q.last_timing(), file=sys.stderr, flush=True)

    torch.cuda.synchronize()
    with GpuTelemetry(enabled=not args.no_telemetry) as telemetry:
        t0 = time.perf_counter()
        kernel_ms, timings, result = [], [], None
        for k in range(args.steps):
            result = q.search(Qd, args.prefix_bits, args.cache_bits, strict=args.strict)
            t = q.last_timing()
            timings.append(t)
            kernel_ms.append(t["search_ms"])
            print("[bench] step", k, t, file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    coverage_ok = all(covers(t, plan["prefix_bits"], plan["suffix_bits"]) for t in timings)

    ms_per_step = elapsed * 1e3 / args.steps
    value = states * args.steps / elapsed / 1e12
    avg_kernel_s = sum(kernel_ms) / len(kernel_ms) / 1e3
    achieved = OPS_PER_STATE * states / avg_kernel_s
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "1e12 states/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": cfg["desc"] + ", seed %d, 2^%d states per step" % (cfg["seed"], n),
                   "name": args.config, "n": n, "states_per_step": states,
                   "prefix_bits": plan["prefix_bits"], "suffix_bits": plan["suffix_bits"],
                   "cache_bits": plan["cache_bits"], "seg_bits": plan["seg_bits"],
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "alu",
            "kernel": "gray_search_kernel<%d, %s>" % (plan["cols_per_lane"], "false" if args.strict else "true"),
            "achieved": achieved / 1e12,
            "peak": INT32_VALU_PEAK / 1e12,
            "unit": "int32 Tops/s",
            "frac": achieved / INT32_VALU_PEAK,
            "traffic": measured_traffic(),
            "ops_per_state": OPS_PER_STATE,
            "peak_derivation": "256 CU x 4 SIMD x 32 lanes/clock x 2.4 GHz (two-operand int32 add)",
            "kernel_ms_avg": avg_kernel_s * 1e3,
            "kernel_timing": "HIP events recorded on the search stream around the kernel launch",
        },
        "pct_int32_valu_peak": 100.0 * value * 1e12 / INT32_VALU_PEAK,
        "result": {"min_energy": result.min_energy, "argmin": result.argmin, "count": result.count},
        "gpu_telemetry": telemetry.summary(),
        "mode": "strict (minimum after every prefix)" if args.strict else
                "bound-gated minimum (one add per state; per-step minimum only where a 32-step bound can reach the best)",
        "coverage_ok": coverage_ok,
        "bodies": timings[-1]["bodies"],
        "checked_bodies": timings[-1]["checked_bodies"],
        "slow_bodies": timings[-1]["slow_bodies"],
        "build_ms_avg": sum(t["build_ms"] for t in timings) / len(timings),
    }
    if not args.strict and not args.no_strict_leg:
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        rs = q.search(Qd, args.prefix_bits, args.cache_bits, strict=True)
        torch.cuda.synchronize()
        ts = q.last_timing()
        line["strict_mode"] = {"value": states / (time.perf_counter() - t1) / 1e12, "unit": "1e12 states/s",
                               "kernel": "gray_search_kernel<%d, false>" % plan["cols_per_lane"],
                               "kernel_ms": ts["search_ms"],
                               "frac": OPS_PER_STATE * states / (ts["search_ms"] / 1e3) / INT32_VALU_PEAK,
                               "ops_per_state_strict": OPS_PER_STATE_STRICT,
                               "frac_add_and_compare": OPS_PER_STATE_STRICT * states / (ts["search_ms"] / 1e3)
                               / INT32_VALU_PEAK,
                               "same_result": rs.triple() == result.triple()}
        print("[bench] strict", ts, file=sys.stderr, flush=True)
    if not args.no_spectrum_leg:
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        low = q.lowest(Qd, 64, args.prefix_bits, args.cache_bits)
        torch.cuda.synchronize()
        tl = q.last_timing()
        line["spectrum_k64"] = {"value": states / (time.perf_counter() - t1) / 1e12, "unit": "1e12 states/s",
                                "kernel": "gray_search_kernel<%d, true, lowest>" % plan["cols_per_lane"],
                                "kernel_ms": tl["search_ms"],
                                "frac": OPS_PER_STATE * states / (tl["search_ms"] / 1e3) / INT32_VALU_PEAK,
                                "slow_bodies": tl["slow_bodies"],
                                "coverage_ok": covers(tl, plan["prefix_bits"], plan["suffix_bits"]),
                                "first": list(low[0]), "last": list(low[-1]),
                                "head_is_min": tuple(low[0]) == (result.min_energy, result.argmin)}
        print("[bench] spectrum", tl, file=sys.stderr, flush=True)
    if not args.no_f64_leg:
        cf = qi.make_config("C4f")
        Qf = torch.tensor(cf["Q"], dtype=torch.float64, device="cuda:0")
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        rf = q.search_f64(Qf)
        torch.cuda.synchronize()
        tf = q.last_timing()
        line["f64_C4f"] = {"value": states / (time.perf_counter() - t1) / 1e12, "unit": "1e12 states/s",
                           "workload": cf["desc"] + ", seed %d" % cf["seed"],
                           "kernel": "gray_search_f64_kernel (int32 walk over rounded scaled tables, "
                                     "binary64 re-evaluation)",
                           "kernel_ms": tf["search_ms"],
                           "frac": OPS_PER_STATE * states / (tf["search_ms"] / 1e3) / INT32_VALU_PEAK,
                           "slow_bodies": tf["slow_bodies"], "candidates": tf["candidates"],
                           "coverage_ok": covers(tf, plan["prefix_bits"], plan["suffix_bits"]),
                           "result": [float.hex(rf.min_energy), rf.argmin, rf.count]}
        print("[bench] f64", tf, file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        lowf = q.lowest(Qf, 64)
        torch.cuda.synchronize()
        tl = q.last_timing()
        line["f64_spectrum_k64"] = {"value": states / (time.perf_counter() - t1) / 1e12, "unit": "1e12 states/s",
                                    "kernel": "gray_search_f64_kernel<lowest> (the 64 lowest binary64 states)",
                                    "kernel_ms": tl["search_ms"],
                                    "frac": OPS_PER_STATE * states / (tl["search_ms"] / 1e3) / INT32_VALU_PEAK,
                                    "slow_bodies": tl["slow_bodies"], "candidates": tl["candidates"],
                                    "first": [float.hex(lowf[0][0]), lowf[0][1]],
                                    "last": [float.hex(lowf[-1][0]), lowf[-1][1]],
                                    "head_is_min": (lowf[0][0], lowf[0][1]) == (rf.min_energy, rf.argmin)}
        print("[bench] f64 spectrum", tl, file=sys.stderr, flush=True)
    if not args.no_config_legs:
        line["other_configs"] = config_legs(q, args.config)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


LEG_CONFIGS = ("C1", "C2", "C2p", "C3", "C5")


def config_legs(q, skip):
    """One whole-space search of each other workload (after one warm-up search
    for the small ones), with its kernel time, rate, the bodies walked exactly
    and the roofline fraction: the gated kernel's time depends on the instance
    (how often a body's bound reaches the best energy).  Results with a stored
    oracle answer (tests/golden/<name>.json) are compared with it."""
    import torch
    import qubo_instances as qi
    legs = {}
    for name in LEG_CONFIGS:
        if name == skip:
            continue
        cfg = qi.make_config(name)
        n = cfg["n"]
        Qd = torch.tensor(cfg["Q"], dtype=torch.int32, device="cuda:0")
        plan = q.make_plan(n)
        if n <= 40:
            q.search(Qd)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r = q.search(Qd)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        t = q.last_timing()
        states = 1 << n
        leg = {"n": n, "seed": cfg["seed"], "value": states / wall / 1e12, "unit": "1e12 states/s",
               "kernel_ms": t["search_ms"], "total_ms": t["total_ms"],
               "kernel_states_per_s": states / (t["search_ms"] / 1e3) / 1e12,
               "frac": OPS_PER_STATE * states / (t["search_ms"] / 1e3) / INT32_VALU_PEAK,
               "bodies": t["bodies"], "slow_bodies": t["slow_bodies"],
               "coverage_ok": covers(t, plan["prefix_bits"], plan["suffix_bits"]),
               "result": list(r.triple())}
        stored = os.path.join(ROOT, "tests", "golden", name + ".json")
        if os.path.exists(stored):
            with open(stored) as f:
                g = json.load(f)
            leg["oracle_result"] = [g["min_energy"], g["argmin"], g["count"]]
            leg["same_as_oracle"] = leg["oracle_result"] == leg["result"] and g["sha256_Q"] == qi.sha256_of(cfg["Q"])
        legs[name] = leg
        print("[bench] config", name, t, file=sys.stderr, flush=True)
    return legs


def split_sweep(q, Qd, cfg, prefixes, caches):
    """One search per (prefix_bits, cache_bits) with 8 columns per lane, and per
    cache_bits with 16 columns per lane at the planner's prefix size.  Splits the
    planner rejects are listed as such.  The result is the same at every split."""
    import torch
    n = cfg["n"]
    states = 1 << n
    default = q.make_plan(n)
    ref = q.search(Qd)  # also the warm-up
    ref_t = q.last_timing()
    points = [(A, l, 8) for A in prefixes for l in caches]
    points += [(default["prefix_bits"], l, 16) for l in caches]
    rows = []
    for A, l, cols in points:
        rec = {"prefix_bits": A, "suffix_bits": n - A, "cache_bits": l, "cols_per_lane": cols}
        if l > A:
            continue
        try:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            r = q.search(Qd, A, l, cols_per_lane=cols)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        except q.QuboError as e:
            rec["rejected"] = q.strerror(e.code)
            print(json.dumps({"sweep_point": rec}), flush=True)
            continue
        t = q.last_timing()
        rec.update({"search_ms": t["search_ms"], "total_ms": t["total_ms"], "wall_ms": wall * 1e3,
                    "kernel_states_per_s": states / (t["search_ms"] / 1e3) / 1e12,
                    "frac": states / (t["search_ms"] / 1e3) / INT32_VALU_PEAK,
                    "slow_bodies": t["slow_bodies"], "same_result": r.triple() == ref.triple()})
        rows.append(rec)
        print(json.dumps({"sweep_point": rec}), flush=True)
    best = min(rows, key=lambda r: r["search_ms"])
    print(json.dumps({"sweep": cfg["name"], "n": n, "states": states,
                      "planner_default": {"prefix_bits": default["prefix_bits"],
                                          "cache_bits": default["cache_bits"],
                                          "cols_per_lane": default["cols_per_lane"],
                                          "search_ms": ref_t["search_ms"]},
                      "best": best, "points": len(rows),
                      "all_same_result": all(r["same_result"] for r in rows),
                      "result": list(ref.triple())}), flush=True)


STEPPED_ABOVE = 50  # larger searches run in steps of about 2^48 states, each printing its progress


def size_scan(q, n_min, n_max):
    """One whole-space search per size n: a symmetric int32 matrix with entries
    uniform in [-100, 100] (seed 6000 + n; P1 times "a uniformly random
    matrix", sec. V.C, with no range or seed given), timed from the call to its
    result, tables and reduction included as in P1's Table IV.  Sizes up to 44
    take the median of three calls after a warm-up, larger ones one call; above
    STEPPED_ABOVE variables the search runs as a sequence of steps
    (qubo_progress_init / qubo_search_step), whose device times are summed."""
    import torch
    import qubo_instances as qi
    for n in range(n_min, n_max + 1):
        Qd = torch.tensor(qi.symmetric_uniform(n, 6000 + n, -100, 100), dtype=torch.int32, device="cuda:0")
        plan = q.make_plan(n)
        A, B = plan["prefix_bits"], plan["suffix_bits"]
        rec = {"n": n, "seed": 6000 + n, "prefix_bits": A, "suffix_bits": B, "states": 1 << n}
        if n <= STEPPED_ABOVE:
            reps = 3 if n <= 44 else 1
            if n <= 44:
                q.search(Qd)
            walls, times = [], []
            for _ in range(reps):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                r = q.search(Qd)
                torch.cuda.synchronize()
                walls.append(time.perf_counter() - t0)
                times.append(q.last_timing())
            i = sorted(range(reps), key=lambda k: walls[k])[reps // 2]
            wall, t = walls[i], times[i]
            rec.update({"calls": reps, "search_ms": t["search_ms"], "build_ms": t["build_ms"],
                        "slow_bodies": t["slow_bodies"], "coverage_ok": covers(t, A, B)})
            result = r.triple()
        else:
            p = q.progress_init(Qd)
            search_ms = build_ms = 0.0
            bodies = slow = steps = 0
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            done = False
            while not done:
                done = q.search_step(Qd, p)
                t = q.last_timing()
                search_ms += t["search_ms"]
                build_ms += t["build_ms"]
                bodies += t["bodies"]
                slow += t["slow_bodies"]
                steps += 1
                print("[sizes] n=%d step %d of %d: %.1f s so far" % (n, steps, p.steps_total,
                                                                   time.perf_counter() - t0),
                      file=sys.stderr, flush=True)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            group = 64 * t["cols_per_lane"]
            cols_padded = -(-(1 << B) // group) * group
            rec.update({"steps": steps, "search_ms": search_ms, "build_ms": build_ms, "slow_bodies": slow,
                        "coverage_ok": bodies * 32 * group == (1 << A) * cols_padded})
            result = p.result().triple()
        rec.update({"wall_s": wall, "states_per_s_1e12": (1 << n) / wall / 1e12,
                    "kernel_states_per_s_1e12": (1 << n) / (rec["search_ms"] / 1e3) / 1e12,
                    "frac": (1 << n) / (rec["search_ms"] / 1e3) / INT32_VALU_PEAK,
                    "result": list(result)})
        print(json.dumps({"size_point": rec}), flush=True)
        del Qd
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
