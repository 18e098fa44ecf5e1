"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every pin is a function of an ``oracle.Oracle`` so that the same checks run on
the default build and on mutant builds (``-DORACLE_MUTATION=k``) in
``test_oracle_mutants.py``, which shows that each planted mistake fails a pin.

Sources of truth used here (none of them is the oracle's own code):
  * hand-worked energies of tiny instances (tests/golden/worked_examples.json);
  * closed forms E(0) = 0, E(e_i) = Q_ii, E(e_i + e_j) = Q_ii + Q_jj + Q_ij + Q_ji;
  * a third, numpy implementation: x^T Q x for all 2^n states (n <= 10);
  * special cases (Q = 0, diagonal Q), the planted-minimiser family, Mattis
    instances with ground energy -n(n-1)/2 and two ground states;
  * the Ising <-> QUBO identity H(s) = E_Q(x) + C (Maltsev et al., sec. I);
  * invariances: relabelling of variables (sec. II.D), change of gauge,
    antisymmetric additions and positive scaling.
"""
from __future__ import annotations

import json
import os
import re

import numpy as np
import pytest

import oracle
import qubo_instances as qi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def numpy_all_states(Q) -> tuple[int, int, int]:
    """(min, argmin, count) from x^T Q x over every state, in numpy (n <= 12)."""
    Q = np.asarray(Q, dtype=np.int64)
    n = Q.shape[0]
    idx = np.arange(1 << n, dtype=np.int64)
    X = ((idx[:, None] >> (n - 1 - np.arange(n))[None, :]) & 1).astype(np.int64)
    E = np.einsum("si,ij,sj->s", X, Q, X)
    m = int(E.min())
    where = np.nonzero(E == m)[0]
    return m, int(where[0]), int(where.size)


def rand_general(n, seed, lo=-100, hi=100):
    return qi.general_uniform(n, seed, lo, hi)


# --------------------------------------------------------------------------- pins

def pin_worked_examples(o: oracle.Oracle):
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        data = json.load(f)
    for ex in data["examples"]:
        Q, n = ex["Q"], len(ex["Q"])
        got = [o.energy(Q, i) for i in range(1 << n)]
        assert got == ex["energies"], ex["name"]
        want = (ex["min"], ex["argmin"], ex["count"])
        assert o.search_direct(Q).triple() == want, ex["name"]
        assert o.search_gray(Q, threads=1).triple() == want, ex["name"]


def pin_closed_forms(o: oracle.Oracle):
    for n, seed in [(1, 2001), (2, 2002), (5, 2003), (13, 2004), (40, 2005), (63, 2006)]:
        Q = rand_general(n, seed, -1000, 1000)
        assert o.energy(Q, 0) == 0
        for i in range(n):
            ei = 1 << (n - 1 - i)
            assert o.energy(Q, ei) == Q[i][i], (n, i)
            for j in range(n):
                if j != i:
                    ej = 1 << (n - 1 - j)
                    assert o.energy(Q, ei | ej) == Q[i][i] + Q[j][j] + Q[i][j] + Q[j][i], (n, i, j)


def pin_numpy_third_implementation(o: oracle.Oracle):
    cases = [(n, 2100 + n, -100, 100) for n in range(1, 11)]
    # small entries make heavy ties, which exercise count and the lowest-index rule
    cases += [(n, 2200 + n, -1, 1) for n in range(2, 11)]
    cases += [(n, 2300 + n, -2, 3) for n in (6, 9, 10)]
    for n, seed, lo, hi in cases:
        Q = rand_general(n, seed, lo, hi)
        want = numpy_all_states(Q)
        assert o.search_direct(Q).triple() == want, (n, seed)
        for threads in (1, 3):
            assert o.search_gray(Q, threads=threads).triple() == want, (n, seed, threads)


def pin_tiers_agree(o: oracle.Oracle):
    for n in range(1, 17):
        Q = rand_general(n, 2400 + n, -50, 50)
        a = o.search_direct(Q)
        b = o.search_gray(Q)
        assert a.triple() == b.triple(), n
    # sub-cubes: fixing the first k variables is the index range [top<<m, (top+1)<<m)
    Q = rand_general(14, 2450, -3, 3)
    for k, top in [(1, 1), (3, 5), (7, 100), (14, 12345)]:
        m = 14 - k
        a = o.search_direct(Q, top << m, (top + 1) << m)
        b = o.search_gray(Q, k, top)
        assert a.triple() == b.triple(), (k, top)


def pin_special_cases(o: oracle.Oracle):
    for n in (1, 4, 11, 16):
        zero = qi.zeros(n)
        assert o.search_gray(zero).triple() == (0, 0, 1 << n)
        assert o.search_direct(zero).triple() == (0, 0, 1 << n)
        pos = qi.zeros(n)
        neg = qi.zeros(n)
        for i in range(n):
            pos[i][i] = 1 + i
            neg[i][i] = -(1 + 2 * i)
        assert o.search_gray(pos).triple() == (0, 0, 1)
        assert o.search_direct(neg).triple() == (sum(neg[i][i] for i in range(n)), (1 << n) - 1, 1)
        assert o.search_gray(neg).triple() == (sum(neg[i][i] for i in range(n)), (1 << n) - 1, 1)


def pin_planted(o: oracle.Oracle):
    for n, seed in [(3, 2501), (8, 2502), (13, 2503), (20, 2504)]:
        Q, P, a = qi.planted(n, seed)
        av = np.asarray(a, dtype=np.int64)
        want_min = -int(av @ np.asarray(P, dtype=np.int64) @ av)
        want = (want_min, qi.bits_to_index(a), 1)
        assert o.search_gray(Q).triple() == want, (n, seed)
        if n <= 13:
            assert o.search_direct(Q).triple() == want, (n, seed)


def pin_mattis(o: oracle.Oracle):
    for n, seed in [(2, 3001), (5, 3002), (12, 3003), (18, 3004)]:
        J, h, xi = qi.mattis(n, seed)
        Q, C = qi.ising_to_qubo(J, h)
        # s = xi and s = -xi; x = (1 + s) / 2.  The lower index has x_0 = 0.
        xa = [(1 + s) // 2 for s in xi]
        xb = [1 - v for v in xa]
        want_arg = min(qi.bits_to_index(xa), qi.bits_to_index(xb))
        r = o.search_gray(Q)
        assert r.min_energy + C == -n * (n - 1) // 2, (n, seed)
        assert (r.argmin, r.count) == (want_arg, 2), (n, seed)


def pin_ising_identity(o: oracle.Oracle):
    for n, seed in [(3, 3101), (7, 3102), (11, 3103)]:
        rng = qi.SplitMix64(seed)
        J = qi.zeros(n)
        for i in range(n):
            for j in range(i + 1, n):
                J[i][j] = rng.uniform_int(-5, 5)
        h = [rng.uniform_int(-5, 5) for _ in range(n)]
        Q, C = qi.ising_to_qubo(J, h)
        idx = np.arange(1 << n, dtype=np.uint64)
        E = o.energies(Q, idx)
        S = 2 * ((idx[:, None].astype(np.int64) >> (n - 1 - np.arange(n))[None, :]) & 1) - 1
        Ju = np.triu(np.asarray(J, dtype=np.int64), 1)
        H = np.einsum("si,ij,sj->s", S, Ju, S) + S @ np.asarray(h, dtype=np.int64)
        assert np.array_equal(H, E + C), (n, seed)


def pin_invariances(o: oracle.Oracle):
    n = 9
    Q = np.asarray(rand_general(n, 3201, -60, 60), dtype=np.int64)
    base = o.search_gray(Q)
    assert base.triple() == o.search_direct(Q).triple()
    # relabelling: x'_i = x_perm[i]
    perm = [3, 0, 8, 5, 1, 7, 2, 6, 4]
    Qp = Q[np.ix_(perm, perm)]
    rp = o.search_gray(Qp)
    assert (rp.min_energy, rp.count) == (base.min_energy, base.count)
    if base.count == 1:
        bits = qi.index_to_bits(base.argmin, n)
        assert rp.argmin == qi.bits_to_index([bits[p] for p in perm])
    # gauge: E_Q'(x) = E_Q(x xor a) - E_Q(a)
    a = [1, 0, 1, 1, 0, 0, 1, 0, 1]
    Qg = qi.gauge_transform(Q.tolist(), a)
    av = np.asarray(a, dtype=np.int64)
    rg = o.search_gray(Qg)
    assert (rg.min_energy, rg.count) == (base.min_energy - int(av @ Q @ av), base.count)
    if base.count == 1:
        assert rg.argmin == base.argmin ^ qi.bits_to_index(a)
    # antisymmetric additions change no energy
    K = np.asarray(rand_general(n, 3202, -30, 30), dtype=np.int64)
    assert o.search_gray(Q + K - K.T).triple() == base.triple()
    assert o.search_direct(Q + K - K.T).triple() == base.triple()
    # positive scaling
    r3 = o.search_gray(3 * Q)
    assert r3.triple() == (3 * base.min_energy, base.argmin, base.count)


def numpy_lowest(Q, k):
    """The k lowest (E, index) pairs of x^T Q x over every state, ordered by E
    then index, from a numpy sort (n <= 12)."""
    Q = np.asarray(Q, dtype=np.int64)
    n = Q.shape[0]
    idx = np.arange(1 << n, dtype=np.int64)
    X = ((idx[:, None] >> (n - 1 - np.arange(n))[None, :]) & 1).astype(np.int64)
    E = np.einsum("si,ij,sj->s", X, Q, X)
    order = np.lexsort((idx, E))[:k]
    return [(int(E[i]), int(i)) for i in order]


def pin_lowest(o: oracle.Oracle):
    """The k lowest states (the low-energy spectrum)."""
    for n, seed, lo, hi in [(1, 2601, -5, 5), (4, 2602, -2, 2), (7, 2603, -1, 1), (9, 2604, -50, 50),
                            (10, 2605, -1, 1), (11, 2606, -3, 3)]:
        Q = rand_general(n, seed, lo, hi)
        for k in (1, 5, 64, (1 << n) + 3):
            k = min(k, 1024)
            want = numpy_lowest(Q, k)
            assert o.lowest(Q, k, gray_walk=True, threads=3) == want, (n, seed, k)
            if n <= 10:
                assert o.lowest(Q, k, gray_walk=False) == want, (n, seed, k)
        # the list begins with every minimiser, in index order
        m = o.search_gray(Q)
        low = o.lowest(Q, min(1 << n, 1024))
        assert low[0] == (m.min_energy, m.argmin), (n, seed)
        assert sum(1 for e, _ in low if e == m.min_energy) == m.count, (n, seed)
    # a sub-cube (first `fixed` variables spell `top`) is the index range [top << m, (top + 1) << m)
    Q = rand_general(12, 2607, -2, 2)
    full = numpy_lowest(Q, 1 << 12)
    for fixed, top in [(1, 1), (3, 5), (6, 40)]:
        m = 12 - fixed
        want = [p for p in full if (p[1] >> m) == top][:40]
        assert o.lowest(Q, 40, gray_walk=True, threads=2, fixed=fixed, top=top) == want, (fixed, top)
        assert o.lowest(Q, 40, gray_walk=False, fixed=fixed, top=top) == want, (fixed, top)
    # Q = 0: every state has E = 0, so the list is the first k indices
    for n in (3, 12):
        assert o.lowest(qi.zeros(n), 8) == [(0, i) for i in range(8)]
    # positive diagonal, no couplings: E is a sum of distinct weights 2^i,
    # so the spectrum is the states ordered by E, each E met once
    n = 6
    pos = qi.zeros(n)
    for i in range(n):
        pos[i][i] = 1 << i          # variable i has weight 2^i -> E = reverse-bit value
    low = o.lowest(pos, 1 << n)
    assert [e for e, _ in low] == list(range(1 << n))
    for e, idx in low:
        assert sum(1 << i for i in range(n) if (idx >> (n - 1 - i)) & 1) == e


# ------------------------------------------------------------------- fp64 pins

def _f(v) -> float:
    return float.fromhex(v) if "0x" in v else float(v)


def pin_f64_worked_examples(o: oracle.Oracle):
    with open(os.path.join(GOLDEN, "worked_examples_f64.json")) as f:
        data = json.load(f)
    for ex in data["examples"]:
        vals = [_f(v) for v in ex["Q"]]
        n = int(round(len(vals) ** 0.5))
        Q = np.asarray(vals, dtype=np.float64).reshape(n, n)
        got = [o.energy_f64(Q, i) for i in range(1 << n)]
        assert got == [_f(v) for v in ex["energies"]], ex["name"]
        want = (_f(ex["min"]), ex["argmin"], ex["count"])
        for threads in (1, 2, 4):
            assert o.search_direct_f64(Q, threads=threads).triple() == want, (ex["name"], threads)


def pin_f64_integer_valued(o: oracle.Oracle):
    """Integer-valued binary64 matrices sum exactly (|partial sums| < 2^53), so
    the floating-point result equals the integer oracle's."""
    for n, seed, lo, hi in [(1, 2701, -5, 5), (6, 2702, -1, 1), (9, 2703, -100, 100), (12, 2704, -2, 2),
                            (14, 2705, -1000, 1000)]:
        Q = rand_general(n, seed, lo, hi)
        r = o.search_direct(Q)
        rf = o.search_direct_f64(np.asarray(Q, dtype=np.float64), threads=3)
        assert rf.triple() == (float(r.min_energy), r.argmin, r.count), (n, seed)
        idx = np.arange(1 << n, dtype=np.uint64)
        assert np.array_equal(o.energies_f64(np.asarray(Q, dtype=np.float64), idx),
                              o.energies(Q, idx).astype(np.float64)), (n, seed)


def pin_f64_fractional(o: oracle.Oracle):
    """Fractional matrices: exact scaling by powers of two, closed forms of
    single-variable states, and a planted instance whose minimiser is known."""
    rng = np.random.default_rng(2711)
    for n in (5, 10, 13):
        Q = rng.uniform(-50.0, 50.0, size=(n, n))
        base = o.search_direct_f64(Q)
        for k in (-3, 1, 7):  # x 2^k is exact in every partial sum
            r = o.search_direct_f64(Q * 2.0 ** k)
            assert r.triple() == (base.min_energy * 2.0 ** k, base.argmin, base.count), (n, k)
        assert o.energy_f64(Q, 0) == 0.0
        for i in range(n):
            assert o.energy_f64(Q, 1 << (n - 1 - i)) == Q[i, i]
    # planted: Q = gauge transform of a positive-definite-like P (integer part)
    # plus tiny fractional noise; the minimiser stays x* (gap >= 1 >> noise)
    Qi, P, a = qi.planted(11, 2712)
    Qf = np.asarray(Qi, dtype=np.float64) + rng.uniform(-1e-3, 1e-3, size=(11, 11))
    r = o.search_direct_f64(Qf)
    av = np.asarray(a, dtype=np.int64)
    assert (r.argmin, r.count) == (qi.bits_to_index(a), 1)
    assert abs(r.min_energy + float(av @ np.asarray(P, dtype=np.int64) @ av)) < 11 * 11 * 1e-3


def pin_f64_lowest(o: oracle.Oracle):
    """The k lowest states of a float64 Q: the sort of all 2^n definition
    energies by (E, index) (numpy's lexsort; the energies are pinned above),
    the integer oracle's list on integer-valued matrices (exact sums, heavy
    ties), the minimum search's head, and index ranges."""
    rng = np.random.default_rng(2721)
    for n in (1, 5, 9, 11):
        for Q in (rng.uniform(-20.0, 20.0, size=(n, n)),
                  np.asarray(rand_general(n, 2722 + n, -2, 2), dtype=np.float64)):
            idx = np.arange(1 << n, dtype=np.uint64)
            E = o.energies_f64(Q, idx)
            order = np.lexsort((idx, E))
            for k in (1, 7, 64, (1 << n) + 3):
                k = min(k, 1024)
                want = [(float(E[i]), int(idx[i])) for i in order[:k]]
                for threads in (1, 3):
                    assert o.lowest_f64(Q, k, threads=threads) == want, (n, k, threads)
            m = o.search_direct_f64(Q)
            low = o.lowest_f64(Q, min(1 << n, 1024))
            assert low[0] == (m.min_energy, m.argmin)
            assert sum(1 for e, _ in low if e == m.min_energy) == m.count
    Qi = rand_general(10, 2723, -1, 1)
    assert o.lowest_f64(np.asarray(Qi, dtype=np.float64), 50) == \
        [(float(e), i) for e, i in o.lowest(Qi, 50)]
    Q = rng.uniform(-5.0, 5.0, size=(12, 12))
    full = o.lowest_f64(Q, 1024)
    for lo, hi in [(0, 64), (100, 1000), (4000, 4096)]:
        assert o.lowest_f64(Q, 20, lo, hi, threads=2) == sorted(
            (o.energy_f64(Q, i), i) for i in range(lo, hi))[:20], (lo, hi)
    assert o.lowest_f64(Q, 20)[:20] == full[:20]


ALL_PINS_F64 = [pin_f64_worked_examples, pin_f64_integer_valued, pin_f64_fractional, pin_f64_lowest]


ALL_PINS = [pin_worked_examples, pin_closed_forms, pin_numpy_third_implementation, pin_tiers_agree,
            pin_special_cases, pin_planted, pin_mattis, pin_ising_identity, pin_invariances,
            pin_lowest]


# -------------------------------------------------------------------------- tests

@pytest.mark.parametrize("pin", ALL_PINS + ALL_PINS_F64, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.default())


def test_fig5_gray_sequence():
    """The binary-reflected Gray code g(i) = i ^ (i >> 1), which orders the
    prefix walk and the prefix-energy table, is the sequence printed in Fig. 5."""
    with open(os.path.join(GOLDEN, "gray_fig5.json")) as f:
        fig = json.load(f)
    b = fig["bits"]
    assert [format(i ^ (i >> 1), "0%db" % b) for i in range(1 << b)] == fig["sequence"]
    # consecutive codes differ in exactly one bit, and the flipped bit is ctz(i+1)
    for i in range((1 << b) - 1):
        d = (i ^ (i >> 1)) ^ ((i + 1) ^ ((i + 1) >> 1))
        assert d == ((i + 1) & -(i + 1))


def test_numpy_reference_itself():
    """The numpy third implementation reproduces the hand-worked energies."""
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        data = json.load(f)
    for ex in data["examples"]:
        assert numpy_all_states(ex["Q"]) == (ex["min"], ex["argmin"], ex["count"])


def test_generators_are_stable():
    """The seeded workloads hash to the values recorded with every stored result
    (whole spaces, sub-cubes, slices and spectra): each stored file names its
    workload by the leading part of its name (C4sub36 -> C4, C2plow -> C2p)."""
    hashes = {}
    checked = set()
    for fname in sorted(os.listdir(GOLDEN)):
        if not fname.endswith(".json"):
            continue
        with open(os.path.join(GOLDEN, fname)) as f:
            rec = json.load(f)
        if "sha256_Q" not in rec:
            continue
        m = re.match(r"C\d+[pf]?", fname)
        assert m, fname
        name = m.group(0)
        if name not in hashes:
            hashes[name] = qi.sha256_of(qi.make_config(name)["Q"])
        assert hashes[name] == rec["sha256_Q"], fname
        checked.add(name)
    # every benchmark workload has stored results to check against
    assert {"C1", "C2", "C2p", "C3", "C4", "C5", "C1f", "C2f", "C4f", "C58"} <= checked, checked


def test_config_families():
    """Structural facts of the workloads, read off the matrices."""
    c3 = qi.make_config("C3")
    Q = np.asarray(c3["Q"])
    off = Q[~np.eye(40, dtype=bool)]
    assert set(np.unique(off)) == {-2, 2}
    assert np.all(Q % 2 == 0) and np.array_equal(Q, Q.T)
    c5 = qi.make_config("C5")
    Q5 = np.asarray(c5["Q"])
    assert np.array_equal(Q5, Q5.T)
    # a rank-4 signal stands out of the noise: four eigenvalues well clear of the rest
    w = np.sort(np.abs(np.linalg.eigvalsh(Q5.astype(float))))[::-1]
    assert w[3] > 2 * w[4]
    for name, (lo, hi) in (("C1", (-100, 100)), ("C4", (-100, 100))):
        Qx = np.asarray(qi.make_config(name)["Q"])
        assert Qx.min() >= lo and Qx.max() <= hi and np.array_equal(Qx, Qx.T)
