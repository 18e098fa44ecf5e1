"""Full-size searches (n = 48 and n = 50) in the benchmark's launch configuration.

A full CPU oracle run at these sizes takes CPU-days, so the answers are checked
with what holds at any size and what the oracle can compute one state at a time:
  * planted and Mattis instances of the same size, whose minimum, minimiser and
    count are known in closed form;
  * E(argmin) == min_energy by the oracle's direct evaluation, and no single
    flip of the minimiser is lower (local optimality of a global minimum);
  * two different kernels (bound-gated with 8 columns per lane, strict with 16)
    return the same triple;
  * every 32-step body was walked (coverage counter).
  * the sub-cube of 2^32 states that holds the reported minimiser (its first
    n - 32 variables fixed to the minimiser's), searched by the oracle here and
    by the library's slice search at the benchmark's split: both give the
    reported minimum and minimiser.
Seeded sub-cubes of the same workloads (2^32 to 2^37 states, and one 2^40-state
slice across several work-unit segments) are compared with stored oracle results
in test_gpu_parity.py.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
import qubo_instances as qi
from gpu_helpers import announce, check_coverage, dev_q, inv_gray

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ising_ground_state_amd as lib
    lib.load()
    return lib


def test_planted_n48(q):
    Q, P, a = qi.planted(48, 8048)
    av = np.asarray(a, dtype=np.int64)
    want = (-int(av @ np.asarray(P, dtype=np.int64) @ av), qi.bits_to_index(a), 1)
    announce("planted n=48")
    assert q.search(dev_q(Q)).triple() == want
    check_coverage(q, 48)


def test_mattis_n48(q):
    J, h, xi = qi.mattis(48, 8148)
    Q, C = qi.ising_to_qubo(J, h)
    xa = [(1 + s) // 2 for s in xi]
    want_arg = min(qi.bits_to_index(xa), qi.bits_to_index([1 - v for v in xa]))
    announce("mattis n=48")
    r = q.search(dev_q(Q))
    assert (r.min_energy + C, r.argmin, r.count) == (-48 * 47 // 2, want_arg, 2)
    check_coverage(q, 48)


def _is_local_min(Q, n, r):
    e = oracle.energy(Q, r.argmin)
    assert e == r.min_energy
    flips = np.asarray([r.argmin ^ (1 << k) for k in range(n)], dtype=np.uint64)
    assert (oracle.energies(Q, flips) >= r.min_energy).all()


@pytest.mark.parametrize("name", ["C4", "C5"])
def test_benchmark_workloads(q, name):
    """The whole space of the n = 48 and n = 50 workloads.  The oracle cannot
    search 2^48 states here, but it searches the 2^32-state sub-cube that holds
    the reported minimiser in seconds: its minimum and lowest minimiser must be
    the reported ones (the minimiser's sub-cube holds the whole space's minimum,
    and the lowest minimiser of the whole space is the lowest of that
    sub-cube's), and the library's slice search of the same sub-cube, at the
    benchmark's split, must return the oracle's triple."""
    cfg = qi.make_config(name)
    n = cfg["n"]
    Qd = dev_q(cfg["Q"])
    announce("full", name, "gated R=8")
    r = q.search(Qd)
    check_coverage(q, n)
    assert r.count >= 1
    _is_local_min(cfg["Q"], n, r)
    if name == "C4":
        announce("full", name, "strict R=16")
        r2 = q.search(Qd, strict=True, cols_per_lane=16)
        check_coverage(q, n, strict=True, cols_per_lane=16)
        assert r2.triple() == r.triple()
    k = n - 32
    top = r.argmin >> 32
    announce("oracle on the minimiser's sub-cube", name, k, top)
    want = oracle.search_gray(cfg["Q"], k=k, top=top)
    assert (want.min_energy, want.argmin) == (r.min_energy, r.argmin)
    assert 1 <= want.count <= r.count
    A = q.make_plan(n)["prefix_bits"]
    m = inv_gray(top)
    lo, hi = m << (A - k), (m + 1) << (A - k)
    announce("slice of the minimiser's sub-cube", name, lo, hi)
    assert q.search_range(Qd, A, lo, hi).triple() == want.triple()
    check_coverage(q, n, A, None, lo, hi)


def test_spectrum_n48(q):
    """The 64 lowest states of the benchmark workload (n = 48), checked by what
    holds at any size: the oracle's energy of every listed state, the order,
    the minimum search's answer at the head, the merge of the two halves of the
    space (two slices, the other kernel build), and closure under single flips:
    a neighbour that precedes a listed state in the (E, index) order must be
    listed too."""
    cfg = qi.make_config("C4")
    Q, n = cfg["Q"], cfg["n"]
    Qd = dev_q(Q)
    announce("full spectrum C4 k=64 R=8")
    low = q.lowest(Qd, 64)
    check_coverage(q, n)
    assert len(low) == 64 and low == sorted(low)
    idx = np.asarray([i for _, i in low], dtype=np.uint64)
    assert oracle.energies(Q, idx).tolist() == [e for e, _ in low]
    r = q.search(Qd)
    assert low[0] == (r.min_energy, r.argmin)
    assert sum(1 for e, _ in low if e == r.min_energy) == min(r.count, 64)
    listed = set(low)
    for e, i in low:
        nb = np.asarray([i ^ (1 << b) for b in range(n)], dtype=np.uint64)
        for e2, i2 in zip(oracle.energies(Q, nb).tolist(), nb.tolist()):
            if (e2, i2) < (e, i):
                assert (e2, i2) in listed, ((e, i), (e2, i2))
    A = q.make_plan(n)["prefix_bits"]
    half = 1 << (A - 1)
    announce("full spectrum C4 halves R=16")
    h0 = q.lowest(Qd, 64, prefix_bits=A, gray_lo=0, gray_hi=half, cols_per_lane=16)
    h1 = q.lowest(Qd, 64, prefix_bits=A, gray_lo=half, gray_hi=2 * half, cols_per_lane=16)
    assert sorted(h0 + h1)[:64] == low


def test_split_invariance_n48(q):
    """The benchmark workload (n = 48) at other prefix/suffix splits and cache
    sizes gives the same triple and the same 64 lowest states: the result
    depends on Q only."""
    cfg = qi.make_config("C4")
    Qd = dev_q(cfg["Q"])
    announce("C4 default split")
    want = q.search(Qd).triple()
    for A, l in [(26, 8), (30, 10), (32, 14)]:
        announce("C4 split", A, l)
        assert q.search(Qd, prefix_bits=A, cache_bits=l).triple() == want, (A, l)
        check_coverage(q, 48, A, l)
    announce("C4 spectrum default split")
    low = q.lowest(Qd, 64)
    announce("C4 spectrum split 31 12")
    assert q.lowest(Qd, 64, prefix_bits=31, cache_bits=12) == low


def test_invariances_full_size(q):
    """The whole n = 48 space (C4) under four changes of the matrix whose effect
    on the result is known: a permutation of the variables (min and count kept,
    the minimiser's bits permuted), an added antisymmetric matrix (nothing
    changes: E depends on Q_ij + Q_ji only), the gauge flip x -> x xor m
    (min - E(m), count kept, argmin xor m) and scaling by 3 (min x 3).  The
    minimiser is unique (count 1), so its index is determined by the map."""
    cfg = qi.make_config("C4")
    n = 48
    Q = np.array(cfg["Q"], dtype=np.int64)
    announce("C4 reference")
    r0 = q.search(dev_q(Q))
    assert r0.count == 1
    x0 = r0.bits(n)
    rng = qi.SplitMix64(9201)
    perm = list(range(n))
    for i in range(n - 1, 0, -1):  # Fisher-Yates
        j = rng.uniform_int(0, i)
        perm[i], perm[j] = perm[j], perm[i]
    Qp = Q[np.ix_(perm, perm)]  # variable i of Qp is variable perm[i] of Q
    announce("C4 permuted")
    rp = q.search(dev_q(Qp))
    assert (rp.min_energy, rp.count) == (r0.min_energy, 1)
    assert rp.bits(n) == [x0[perm[i]] for i in range(n)]
    S = np.zeros((n, n), dtype=np.int64)
    for i in range(n):
        for j in range(i + 1, n):
            S[i, j] = rng.uniform_int(-100, 100)
            S[j, i] = -S[i, j]
    announce("C4 plus antisymmetric")
    assert q.search(dev_q(Q + S)).triple() == r0.triple()
    mask = [rng.uniform_int(0, 1) for _ in range(n)]
    m = qi.bits_to_index(mask)
    Qg = np.array(qi.gauge_transform(Q.tolist(), mask), dtype=np.int64)
    announce("C4 gauge flip")
    rg = q.search(dev_q(Qg))
    assert rg.triple() == (r0.min_energy - oracle.energy(Q.tolist(), m), r0.argmin ^ m, 1)
    announce("C4 times 3")
    assert q.search(dev_q(3 * Q)).triple() == (3 * r0.min_energy, r0.argmin, 1)


def test_largest_single_launch_n58(q):
    """n = 58, the largest size one launch searches: the planner's split is
    A = 32, B = 26 (a 16 GiB prefix table and 8 GiB of M_int, at the caps).
    Seeded slices of 2^36 states against stored oracle results
    (tests/golden/C58sub.json): minimum, count and index, and the 16 lowest."""
    path = os.path.join(os.path.dirname(__file__), "golden", "C58sub.json")
    if not os.path.exists(path):
        pytest.skip("stored oracle result C58sub.json not written yet")
    with open(path) as f:
        g = json.load(f)
    cfg = qi.make_config("C58")
    assert qi.sha256_of(cfg["Q"]) == g["sha256_Q"]
    plan = q.make_plan(58)
    A = plan["prefix_bits"]
    assert (A, plan["suffix_bits"]) == (32, 26)
    Qd = dev_q(cfg["Q"])
    for cube in g["cubes"]:
        k, top = cube["k"], cube["top"]
        m = inv_gray(top)
        lo, hi = m << (A - k), (m + 1) << (A - k)
        announce("n=58 slice", k, top)
        r = q.search_range(Qd, A, lo, hi)
        assert r.triple() == (cube["min_energy"], cube["argmin"], cube["count"]), top
        check_coverage(q, 58, A, None, lo, hi)
        if "lowest16" in cube:
            announce("n=58 slice lowest", k, top)
            low = q.lowest(Qd, 16, prefix_bits=A, gray_lo=lo, gray_hi=hi)
            assert low == [(int(e), int(i)) for e, i in cube["lowest16"]]


def test_largest_single_launch_n58_f64(q):
    """The binary64 search at n = 58 (A = 32, B = 26: its rounded walk at the
    largest tables): C58 as binary64 with pi added to Q_00, so the matrix is not
    dyadic and the search takes the rounded walk.  Every state of the stored
    slices has x_0 = 0, where the sums never meet Q_00 and are exact integers,
    so the slices' binary64 minima, indices, counts and 16 lowest states are
    the stored integer oracle results."""
    import torch
    path = os.path.join(os.path.dirname(__file__), "golden", "C58sub.json")
    if not os.path.exists(path):
        pytest.skip("stored oracle result C58sub.json not written yet")
    with open(path) as f:
        g = json.load(f)
    cfg = qi.make_config("C58")
    assert qi.sha256_of(cfg["Q"]) == g["sha256_Q"]
    Qf = np.asarray(cfg["Q"], dtype=np.float64)
    Qf[0, 0] += np.pi
    with pytest.raises(q.QuboError):
        q.f64_as_int32(Qf)  # not dyadic: the rounded walk runs
    A = q.make_plan(58)["prefix_bits"]
    Qd = torch.as_tensor(Qf).to("cuda:0").contiguous()
    for cube in g["cubes"]:
        k, top = cube["k"], cube["top"]
        assert top >> (k - 1) == 0  # variable 0 is 0 in the slice
        m = inv_gray(top)
        lo, hi = m << (A - k), (m + 1) << (A - k)
        announce("n=58 binary64 slice", k, top)
        r = q.search_f64(Qd, prefix_bits=A, gray_lo=lo, gray_hi=hi)
        assert r.triple() == (float(cube["min_energy"]), cube["argmin"], cube["count"]), top
        assert q.last_timing()["candidates"] > 0
        check_coverage(q, 58, A, None, lo, hi)
        if "lowest16" in cube:
            announce("n=58 binary64 slice lowest", k, top)
            low = q.lowest(Qd, 16, prefix_bits=A, gray_lo=lo, gray_hi=hi)
            assert low == [(float(e), int(i)) for e, i in cube["lowest16"]]
    del Qd
    torch.cuda.synchronize()
