"""Write the stored oracle results under tests/golden/.

Calls only the CPU oracle (``oracle``) on the seeded workloads of
``qubo_instances``; nothing here comes from the solver.  Usage:

    python tests/golden/make_golden.py C1 C2 C2p        # full searches
    python tests/golden/make_golden.py C3               # 2^40 states, ~25 min on 8 cores
    python tests/golden/make_golden.py C4sub C5sub      # seeded sub-cubes of 2^32 states
    python tests/golden/make_golden.py C1low C2low C2plow C4sublow C5sublow
                                                        # the 64 lowest states (spectrum)
    python tests/golden/make_golden.py C1f C2f C4fsub   # real-valued (binary64) workloads, tier A
    python tests/golden/make_golden.py C58sub           # n = 58 (largest single launch): 2^36-state sub-cubes
    python tests/golden/make_golden.py C1flow C4fsublow # binary64 spectrum: whole C1f, two C4f sub-cubes
    python tests/golden/make_golden.py C4sub36 C5sub37  # deeper sub-cubes: 2^36 (n=48) and 2^37 (n=50) states
    python tests/golden/make_golden.py C4slice          # 8 consecutive 2^37-state sub-cubes of n=48 (2^40 states)

Full searches store {sha256_Q, n, min_energy, argmin, count, max_abs_energy}.
Sub-cube files store one record per sub-cube: the first k variables are fixed
to `top` (variable 0 most significant) and the remaining 32 are searched.
Spectrum files (names ending in "low") store the first 64 states in the order
(E ascending, index ascending) of the whole space or of each sub-cube.
"""
from __future__ import annotations

import json
import os
import platform
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import qubo_instances as qi  # noqa: E402

SUB_FREE_BITS = 32
SUB_COUNT = 16
SUB_SEED = 4242


def host_info(threads: int) -> dict:
    return dict(threads=threads, cpu=platform.processor() or platform.machine(),
                nproc=os.cpu_count(), oracle=oracle.version())


def full(name: str, threads: int) -> dict:
    cfg = qi.make_config(name)
    Q, n = cfg["Q"], cfg["n"]
    t0 = time.time()
    b = oracle.search_gray(Q, threads=threads)
    tb = time.time() - t0
    rec = dict(name=name, desc=cfg["desc"], n=n, seed=cfg["seed"], sha256_Q=qi.sha256_of(Q),
               min_energy=b.min_energy, argmin=b.argmin, count=b.count,
               max_abs_energy=b.max_abs_energy, tier="B (Gray walk)", seconds_tier_b=round(tb, 2),
               host=host_info(threads))
    if n <= 32:
        t0 = time.time()
        a = oracle.search_direct(Q, threads=threads)
        rec["seconds_tier_a"] = round(time.time() - t0, 2)
        if a.triple() != b.triple():
            raise SystemExit("tier A %s != tier B %s on %s" % (a.triple(), b.triple(), name))
        rec["tier"] = "A (direct) and B (Gray walk), identical"
    if "C" in cfg:
        rec["ising_constant_C"] = cfg["C"]
        rec["ising_min_H"] = b.min_energy + cfg["C"]
    return rec


def subcubes(name: str, threads: int) -> dict:
    cfg = qi.make_config(name)
    Q, n = cfg["Q"], cfg["n"]
    k = n - SUB_FREE_BITS
    cubes = []
    t_all = time.time()
    for top in sub_tops(n):
        t0 = time.time()
        r = oracle.search_gray(Q, k=k, top=top, threads=threads)
        cubes.append(dict(k=k, top=top, min_energy=r.min_energy, argmin=r.argmin, count=r.count,
                          max_abs_energy=r.max_abs_energy, seconds=round(time.time() - t0, 2)))
        print("  %s top=%d -> %s" % (name, top, r.triple()), flush=True)
    return dict(name=name + "sub", desc=cfg["desc"], n=n, seed=cfg["seed"], sha256_Q=qi.sha256_of(Q),
                free_bits=SUB_FREE_BITS, sub_seed=SUB_SEED + n, cubes=cubes, tier="B (Gray walk)",
                seconds_total=round(time.time() - t_all, 2), host=host_info(threads))


LOW_K = 64


def sub_tops(n: int) -> list[int]:
    k = n - SUB_FREE_BITS
    rng = qi.SplitMix64(SUB_SEED + n)
    tops = []
    while len(tops) < SUB_COUNT:
        t = rng.uniform_int(0, (1 << k) - 1)
        if t not in tops:
            tops.append(t)
    return tops


def lowest_full(name: str, threads: int) -> dict:
    cfg = qi.make_config(name)
    Q, n = cfg["Q"], cfg["n"]
    t0 = time.time()
    low = oracle.lowest(Q, LOW_K, gray_walk=True, threads=threads)
    return dict(name=name + "low", desc=cfg["desc"], n=n, seed=cfg["seed"], sha256_Q=qi.sha256_of(Q),
                k=LOW_K, states=[list(p) for p in low], tier="B (Gray walk)",
                seconds=round(time.time() - t0, 2), host=host_info(threads))


def lowest_subcubes(name: str, threads: int) -> dict:
    cfg = qi.make_config(name)
    Q, n = cfg["Q"], cfg["n"]
    k = n - SUB_FREE_BITS
    cubes = []
    t_all = time.time()
    for top in sub_tops(n):
        low = oracle.lowest(Q, LOW_K, gray_walk=True, threads=threads, fixed=k, top=top)
        cubes.append(dict(k=k, top=top, states=[list(p) for p in low]))
        print("  %s top=%d -> %s" % (name, top, low[0]), flush=True)
    return dict(name=name + "sublow", desc=cfg["desc"], n=n, seed=cfg["seed"], sha256_Q=qi.sha256_of(Q),
                free_bits=SUB_FREE_BITS, sub_seed=SUB_SEED + n, k_lowest=LOW_K, cubes=cubes,
                tier="B (Gray walk)", seconds_total=round(time.time() - t_all, 2), host=host_info(threads))


F_SUB_FREE_BITS = 28
F_SUB_COUNT = 8


def full_f64(name: str, threads: int) -> dict:
    cfg = qi.make_config(name)
    Q, n = cfg["Q"], cfg["n"]
    t0 = time.time()
    r = oracle.search_direct_f64(Q, threads=threads)
    return dict(name=name, desc=cfg["desc"], n=n, seed=cfg["seed"], sha256_Q=qi.sha256_of(Q),
                min_energy_hex=float.hex(r.min_energy), min_energy=r.min_energy, argmin=r.argmin,
                count=r.count, tier="A (direct, binary64 in row-major order)",
                seconds=round(time.time() - t0, 2), host=host_info(threads))


def subcubes_f64(name: str, threads: int) -> dict:
    cfg = qi.make_config(name)
    Q, n = cfg["Q"], cfg["n"]
    k = n - F_SUB_FREE_BITS
    rng = qi.SplitMix64(SUB_SEED + 100 + n)
    tops = []
    while len(tops) < F_SUB_COUNT:
        t = rng.uniform_int(0, (1 << k) - 1)
        if t not in tops:
            tops.append(t)
    cubes = []
    t_all = time.time()
    m = F_SUB_FREE_BITS
    for top in tops:
        r = oracle.search_direct_f64(Q, top << m, (top + 1) << m, threads=threads)
        cubes.append(dict(k=k, top=top, min_energy_hex=float.hex(r.min_energy), min_energy=r.min_energy,
                          argmin=r.argmin, count=r.count))
        print("  %s top=%d -> %s" % (name, top, r.triple()), flush=True)
    return dict(name=name + "sub", desc=cfg["desc"], n=n, seed=cfg["seed"], sha256_Q=qi.sha256_of(Q),
                free_bits=F_SUB_FREE_BITS, sub_seed=SUB_SEED + 100 + n, cubes=cubes,
                tier="A (direct, binary64 in row-major order)", seconds_total=round(time.time() - t_all, 2),
                host=host_info(threads))


F_LOW_CUBES = 2


def lowest_full_f64(name: str, threads: int) -> dict:
    cfg = qi.make_config(name)
    Q, n = cfg["Q"], cfg["n"]
    t0 = time.time()
    low = oracle.lowest_f64(Q, 64, threads=threads)
    return dict(name=name + "low", desc=cfg["desc"], n=n, seed=cfg["seed"], sha256_Q=qi.sha256_of(Q), k=64,
                states=[[float.hex(e), i] for e, i in low], tier="A (direct, binary64 in row-major order)",
                seconds=round(time.time() - t0, 2), host=host_info(threads))


def lowest_subcubes_f64(name: str, threads: int) -> dict:
    """The 64 lowest states of the first sub-cubes of the binary64 sub-cube set."""
    sub = subcubes_f64_tops(name)
    cfg = qi.make_config(name)
    Q, n = cfg["Q"], cfg["n"]
    m = F_SUB_FREE_BITS
    cubes = []
    t_all = time.time()
    for top in sub[:F_LOW_CUBES]:
        low = oracle.lowest_f64(Q, 64, top << m, (top + 1) << m, threads=threads)
        cubes.append(dict(k=n - m, top=top, states=[[float.hex(e), i] for e, i in low]))
        print("  %s top=%d -> %s" % (name, top, low[0]), flush=True)
    return dict(name=name + "sublow", desc=cfg["desc"], n=n, seed=cfg["seed"], sha256_Q=qi.sha256_of(Q),
                free_bits=m, sub_seed=SUB_SEED + 100 + n, k_lowest=64, cubes=cubes,
                tier="A (direct, binary64 in row-major order)", seconds_total=round(time.time() - t_all, 2),
                host=host_info(threads))


def subcubes_f64_tops(name: str) -> list[int]:
    """The seeded sub-cube tops of the binary64 sub-cube set (as in subcubes_f64)."""
    n = qi.make_config(name)["n"]
    k = n - F_SUB_FREE_BITS
    rng = qi.SplitMix64(SUB_SEED + 100 + n)
    tops = []
    while len(tops) < F_SUB_COUNT:
        t = rng.uniform_int(0, (1 << k) - 1)
        if t not in tops:
            tops.append(t)
    return tops


MAX_SUB_FREE_BITS = 36
MAX_SUB_COUNT = 2


def subcubes_max(name: str, threads: int) -> dict:
    """Sub-cubes of 2^36 states of the n = 58 workload, with the first 22
    variables fixed, for the minimum, and the 16 lowest states of the first."""
    cfg = qi.make_config(name)
    Q, n = cfg["Q"], cfg["n"]
    k = n - MAX_SUB_FREE_BITS
    rng = qi.SplitMix64(SUB_SEED + 200 + n)
    tops = []
    while len(tops) < MAX_SUB_COUNT:
        t = rng.uniform_int(0, (1 << k) - 1)
        if t not in tops:
            tops.append(t)
    cubes = []
    t_all = time.time()
    for i, top in enumerate(tops):
        r = oracle.search_gray(Q, k=k, top=top, threads=threads)
        cube = dict(k=k, top=top, min_energy=r.min_energy, argmin=r.argmin, count=r.count)
        if i == 0:
            cube["lowest16"] = [list(p) for p in oracle.lowest(Q, 16, gray_walk=True, threads=threads,
                                                                 fixed=k, top=top)]
        cubes.append(cube)
        print("  %s top=%d -> %s" % (name, top, r.triple()), flush=True)
    return dict(name=name + "sub", desc=cfg["desc"], n=n, seed=cfg["seed"], sha256_Q=qi.sha256_of(Q),
                free_bits=MAX_SUB_FREE_BITS, sub_seed=SUB_SEED + 200 + n, cubes=cubes, tier="B (Gray walk)",
                seconds_total=round(time.time() - t_all, 2), host=host_info(threads))


DEEP_COUNT = {"C4": 4, "C5": 3}


def subcubes_deep(name: str, free: int, threads: int) -> dict:
    """Sub-cubes of 2^free states (the first n - free variables fixed): with the
    prefix walked over 28 variables they span 2^(28 - n + free) Gray steps, so
    the walk flips prefix variables far above the low ones."""
    cfg = qi.make_config(name)
    Q, n = cfg["Q"], cfg["n"]
    k = n - free
    rng = qi.SplitMix64(SUB_SEED + 300 + free + n)
    tops = []
    while len(tops) < DEEP_COUNT[name]:
        t = rng.uniform_int(0, (1 << k) - 1)
        if t not in tops:
            tops.append(t)
    cubes = []
    t_all = time.time()
    for top in tops:
        t0 = time.time()
        r = oracle.search_gray(Q, k=k, top=top, threads=threads)
        cubes.append(dict(k=k, top=top, min_energy=r.min_energy, argmin=r.argmin, count=r.count,
                          max_abs_energy=r.max_abs_energy, seconds=round(time.time() - t0, 2)))
        print("  %s top=%d -> %s" % (name, top, r.triple()), flush=True)
    return dict(name="%ssub%d" % (name, free), desc=cfg["desc"], n=n, seed=cfg["seed"],
                sha256_Q=qi.sha256_of(Q), free_bits=free, sub_seed=SUB_SEED + 300 + free + n, cubes=cubes,
                tier="B (Gray walk)", seconds_total=round(time.time() - t_all, 2), host=host_info(threads))


SLICE_K = 11
SLICE_CUBES = 8


def long_slice(name: str, threads: int) -> dict:
    """SLICE_CUBES sub-cubes with the first SLICE_K variables fixed whose values
    are g(j) for SLICE_CUBES consecutive j, starting at an odd j (seeded): the
    union of the ranges [j 2^(A-k), (j+1) 2^(A-k)) of any A-variable prefix walk,
    so one contiguous Gray range.  Each cube's result, and the combination of
    all of them by the rule of the final reduction (minimum, count at the
    minimum, lowest index)."""
    cfg = qi.make_config(name)
    Q, n = cfg["Q"], cfg["n"]
    k = SLICE_K
    rng = qi.SplitMix64(SUB_SEED + 400 + n)
    j0 = 2 * rng.uniform_int(0, ((1 << k) - SLICE_CUBES - 1) // 2) + 1
    cubes = []
    best = None
    t_all = time.time()
    for j in range(j0, j0 + SLICE_CUBES):
        top = j ^ (j >> 1)
        t0 = time.time()
        r = oracle.search_gray(Q, k=k, top=top, threads=threads)
        cubes.append(dict(k=k, j=j, top=top, min_energy=r.min_energy, argmin=r.argmin, count=r.count,
                          seconds=round(time.time() - t0, 2)))
        print("  %s j=%d top=%d -> %s" % (name, j, top, r.triple()), flush=True)
        if best is None or r.min_energy < best[0]:
            best = [r.min_energy, r.argmin, r.count]
        elif r.min_energy == best[0]:
            best = [best[0], min(best[1], r.argmin), best[2] + r.count]
    return dict(name=name + "slice", desc=cfg["desc"], n=n, seed=cfg["seed"], sha256_Q=qi.sha256_of(Q),
                k=k, j_first=j0, cubes_in_slice=SLICE_CUBES, slice_seed=SUB_SEED + 400 + n, cubes=cubes,
                min_energy=best[0], argmin=best[1], count=best[2], tier="B (Gray walk)",
                seconds_total=round(time.time() - t_all, 2), host=host_info(threads))


def main(argv):
    threads = oracle.default_threads()
    for arg in argv:
        print("computing", arg, "on", threads, "threads", flush=True)
        if arg in ("C4sub36", "C5sub37"):
            rec = subcubes_deep(arg[:2], int(arg[5:]), threads)
        elif arg == "C4slice":
            rec = long_slice("C4", threads)
        elif arg == "C58sub":
            rec = subcubes_max("C58", threads)
        elif arg == "C1flow":
            rec = lowest_full_f64("C1f", threads)
        elif arg == "C4fsublow":
            rec = lowest_subcubes_f64("C4f", threads)
        elif arg.endswith("fsub"):
            rec = subcubes_f64(arg[:-3], threads)
        elif arg in ("C1f", "C2f"):
            rec = full_f64(arg, threads)
        elif arg.endswith("sublow"):
            rec = lowest_subcubes(arg[:-6], threads)
        elif arg.endswith("low"):
            rec = lowest_full(arg[:-3], threads)
        elif arg.endswith("sub"):
            rec = subcubes(arg[:-3], threads)
        else:
            rec = full(arg, threads)
        path = os.path.join(HERE, arg + ".json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print("wrote", path, {k: rec[k] for k in rec if k in ("min_energy", "argmin", "count", "seconds")},
              flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["C1", "C2", "C2p"])
