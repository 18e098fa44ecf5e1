"""Parity of the real-valued (binary64) search, qubo_search_f64, with the oracle.

The result is defined as the minimum of the binary64 energy summed in
row-major order over the set variables (the oracle's fp64 tier A), its lowest
minimiser and the number of states with exactly that energy, so the bar is
bit-exact: the same float, index and count as the oracle.
"""
from __future__ import annotations

import ctypes
import json
import os

import numpy as np
import pytest

import oracle
import qubo_instances as qi
from gpu_helpers import announce, check_coverage, gray, inv_gray

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def q():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ising_ground_state_amd as lib
    lib.load()
    return lib


def dev_f(Q):
    import torch
    return torch.as_tensor(np.asarray(Q, dtype=np.float64)).to("cuda:0").contiguous()


def golden(name):
    path = os.path.join(GOLDEN, name + ".json")
    if not os.path.exists(path):
        pytest.skip("stored oracle result %s.json not written yet" % name)
    with open(path) as f:
        return json.load(f)


def real_matrix(n, seed, scale=100.0):
    rng = np.random.default_rng(seed)
    return rng.uniform(-scale, scale, size=(n, n))


@pytest.mark.parametrize("n", list(range(1, 21)))
def test_small_real(q, n):
    Q = real_matrix(n, 8000 + n)
    want = oracle.search_direct_f64(Q).triple()
    announce("f64 small", n)
    assert q.search_f64(dev_f(Q)).triple() == want


@pytest.mark.parametrize("n,seed,lo,hi", [(6, 8101, -1, 1), (11, 8102, -2, 2), (14, 8103, -1, 1),
                                          (16, 8104, -100, 100)])
def test_integer_valued_ties(q, n, seed, lo, hi):
    """Integer-valued matrices (exact sums, many exact ties) give the integer
    oracle's answer, count included."""
    Qi = qi.general_uniform(n, seed, lo, hi)
    want = oracle.search_gray(Qi).triple()
    announce("f64 int-valued", n, seed)
    r = q.search_f64(dev_f(Qi))
    assert (r.min_energy, r.argmin, r.count) == (float(want[0]), want[1], want[2])


def test_mixed_magnitudes(q):
    """Entries spanning 16 decades: the rounded tables (17 significant bits of
    S) cannot rank the states, the re-evaluation against the definition must."""
    rng = np.random.default_rng(8201)
    n = 13
    Q = rng.uniform(-1.0, 1.0, size=(n, n)) * 10.0 ** rng.integers(-8, 8, size=(n, n))
    want = oracle.search_direct_f64(Q).triple()
    announce("f64 mixed magnitudes")
    assert q.search_f64(dev_f(Q)).triple() == want
    # the summation-order example: 1e16 + 1 rounds back to 1e16
    Q2 = np.array([[1e16, 1.0], [-1e16, 0.0]])
    announce("f64 order example")
    assert q.search_f64(dev_f(Q2)).triple() == oracle.search_direct_f64(Q2).triple() == (0.0, 0, 3)


@pytest.mark.parametrize("n", [5, 14])
def test_every_split_real(q, n):
    Q = real_matrix(n, 8300 + n, 10.0)
    want = oracle.search_direct_f64(Q).triple()
    Qd = dev_f(Q)
    for A in range(5, n + 1):
        for l in sorted({5, (5 + A) // 2, A}):
            announce("f64 split", n, A, l)
            assert q.search_f64(Qd, prefix_bits=A, cache_bits=l).triple() == want, (A, l)
            check_coverage(q, n, A, l)


@pytest.mark.parametrize("case", ["normal", "subnormal"])
def test_near_the_floor(q, case):
    """S = sum |Q_ij| just above the guard's floor 2^-100, so the walk's scale
    factor is 2^117.  'normal': entries of one magnitude (about 2^-107).
    'subnormal': every entry but one 36 binary orders below S (2^-136, below
    fp32's normal range), so the rounded tables hold them as 0 and only the
    re-evaluation ranks the states; one diagonal entry lifts S above the floor.
    The minimum, its lowest index, the count and the 16 lowest states equal the
    oracle's binary64 definition."""
    n = 14
    rng = np.random.default_rng(8701 if case == "normal" else 8702)
    Q = rng.uniform(-1.0, 1.0, size=(n, n))
    if case == "normal":
        Q *= 1.5 * 2.0 ** -100 / np.abs(Q).sum()
    else:
        Q *= 2.0 ** -136
        Q[3, 3] = -(2.0 ** -100)
    q.check_q_f64(Q)
    Qd = dev_f(Q)
    announce("f64 near the floor", case)
    assert q.search_f64(Qd).triple() == oracle.search_direct_f64(Q).triple()
    announce("f64 near the floor lowest", case)
    assert q.lowest(Qd, 16) == oracle.lowest_f64(Q, 16)


def test_ties_below_the_quantum(q):
    """An integer-valued matrix (many exact ties) with diagonal perturbations
    of about 2^-30: the states the perturbations separate are 2^21 times closer
    than one unit of the rounded walk (S / 2^17), so the walk sees them as ties
    and only the re-evaluation from the definition ranks them.  Minimum, lowest
    minimiser, count and the 32 lowest states against the oracle."""
    n = 16
    Qi = np.array(qi.general_uniform(n, 8901, -3, 3), dtype=np.float64)
    rng = np.random.default_rng(8902)
    Q = Qi + np.diag(rng.uniform(-1.0, 1.0, size=n) * 2.0 ** -30)
    Qd = dev_f(Q)
    announce("f64 ties below the quantum")
    assert q.search_f64(Qd).triple() == oracle.search_direct_f64(Q).triple()
    announce("f64 ties below the quantum, lowest")
    assert q.lowest(Qd, 32) == oracle.lowest_f64(Q, 32)
    # integer-valued with exact ties: the count runs over the tied states
    announce("f64 integer-valued ties, small entries")
    assert q.search_f64(dev_f(Qi)).triple() == oracle.search_direct_f64(Qi).triple()


def test_entries_below_the_quantum(q):
    """One large diagonal entry and the rest about 10^12 times smaller: the
    rounded tables hold the small entries as 0, so every state without the
    large variable has the same walked value and is re-evaluated (2^11 of
    them); the result still equals the definition's."""
    n = 12
    rng = np.random.default_rng(8903)
    Q = rng.uniform(-1.0, 1.0, size=(n, n)) * 1e-9
    Q[0, 0] = 1e3
    Qd = dev_f(Q)
    announce("f64 entries below the quantum")
    assert q.search_f64(Qd).triple() == oracle.search_direct_f64(Q).triple()
    announce("f64 entries below the quantum, lowest")
    assert q.lowest(Qd, 16) == oracle.lowest_f64(Q, 16)


def test_dyadic_takes_the_integer_search(q):
    """Entries in {-1/8, 0, 1/8} (exact ties, two minimisers): every partial sum
    of the definition is exact, so the search runs as the integer search of 8 Q
    (no state is re-evaluated) and gives the definition's minimum, count and
    lowest states."""
    n = 16
    Q = np.array(qi.general_uniform(n, 8904, -1, 1), dtype=np.float64) / 8.0
    Qd = dev_f(Q)
    announce("f64 dyadic")
    r = q.search_f64(Qd)
    assert q.last_timing()["candidates"] == 0
    assert r.triple() == oracle.search_direct_f64(Q).triple()
    assert r.count > 1
    announce("f64 dyadic lowest")
    assert q.lowest(Qd, 32) == oracle.lowest_f64(Q, 32)
    # the zero matrix: every one of the 2^36 states is a minimiser
    announce("f64 zero n=36")
    assert q.search_f64(dev_f(np.zeros((36, 36)))).triple() == (0.0, 0, 1 << 36)


def test_exact_ties_on_the_rounded_walk(q):
    """An integer-valued matrix with exact ties plus one variable whose
    diagonal (1000 + pi) is not dyadic: the search takes the rounded walk, the
    tied states pass the filter together, and the count of exact ties comes
    from the re-evaluation."""
    n = 15
    Qi = np.array(qi.general_uniform(n, 8905, -1, 1), dtype=np.float64)
    Q = np.zeros((n + 1, n + 1))
    Q[1:, 1:] = Qi
    Q[0, 0] = 1000.0 + np.pi
    Qd = dev_f(Q)
    announce("f64 exact ties, rounded walk")
    r = q.search_f64(Qd)
    assert q.last_timing()["candidates"] > 0
    want = oracle.search_direct_f64(Q).triple()
    assert r.triple() == want and want[2] > 1
    announce("f64 exact ties, rounded walk, lowest")
    assert q.lowest(Qd, 48) == oracle.lowest_f64(Q, 48)


def _real_family(kind, n, rng):
    if kind == "uniform":
        return rng.uniform(-1.0, 1.0, size=(n, n))
    if kind == "log-uniform":  # magnitudes over twelve decades, random signs
        return rng.choice([-1.0, 1.0], size=(n, n)) * 10.0 ** rng.uniform(-6, 6, size=(n, n))
    if kind == "near-ties":  # small integers plus relative noise of 1e-12
        Qi = rng.integers(-2, 3, size=(n, n)).astype(np.float64)
        return Qi * (1.0 + 1e-12 * rng.standard_normal(size=(n, n)))
    if kind == "sparse":  # nine entries in ten are zero
        return rng.uniform(-5.0, 5.0, size=(n, n)) * (rng.random(size=(n, n)) < 0.1)
    if kind == "low-rank":  # a rank-2 product: many near-degenerate states
        u = rng.standard_normal(size=(n, 2))
        return u @ u.T * np.pi
    if kind == "heavy-tail":  # Cauchy entries: a few dominate S
        return rng.standard_cauchy(size=(n, n))
    if kind == "negative":  # every entry <= 0: the tables' offsets are as large as S allows
        return -rng.uniform(0.0, 1.0, size=(n, n))
    if kind == "negative-log":  # and over twelve decades: offsets at the widest rounding (28 bits)
        return -(10.0 ** rng.uniform(-6, 6, size=(n, n)))
    raise KeyError(kind)


FAMILIES = ["uniform", "log-uniform", "near-ties", "sparse", "low-rank", "heavy-tail", "negative",
            "negative-log"]


@pytest.mark.parametrize("kind", FAMILIES)
def test_random_real_families(q, kind):
    """Seeded families of real matrices that stress the rounded walk in
    different ways (entries far below its 17-bit unit, ties broken below the
    unit, zero rows, near-degenerate spectra, a few dominant entries, entries
    of one sign), at n = 8..16: minimum, lowest index, count and the 8 lowest
    states against the oracle's binary64 definition."""
    rng = np.random.default_rng(9900 + FAMILIES.index(kind))
    for n in (8, 11, 13, 16):
        for rep in range(2):
            Q = _real_family(kind, n, rng)
            q.check_q_f64(Q)
            Qd = dev_f(Q)
            announce("f64 family", kind, n, rep)
            assert q.search_f64(Qd).triple() == oracle.search_direct_f64(Q).triple(), (kind, n, rep)
            assert q.lowest(Qd, 8) == oracle.lowest_f64(Q, 8), (kind, n, rep)


def test_one_dominant_entry(q):
    """Entries uniform in [-1e-3, 1e-3] and one diagonal entry of 1e3: with the
    walk's 17-bit tables the small entries would round to a quantum or two and
    about 2^(n-1) states would share a walked value; the rounding widens to
    the small entries' scale (up to 28 bits), the states stay ranked and only a
    handful are re-evaluated.  Result against the oracle."""
    n = 24
    rng = np.random.default_rng(8906)
    Q = rng.uniform(-1.0, 1.0, size=(n, n)) * 1e-3
    Q[0, 0] = 1e3
    Qd = dev_f(Q)
    announce("f64 one dominant entry")
    assert q.search_f64(Qd).triple() == oracle.search_direct_f64(Q).triple()
    assert q.last_timing()["candidates"] < 1000
    announce("f64 one dominant entry, lowest")
    assert q.lowest(Qd, 16) == oracle.lowest_f64(Q, 16)


def test_zero_and_diagonal(q):
    announce("f64 zero")
    assert q.search_f64(dev_f(np.zeros((8, 8)))).triple() == (0.0, 0, 256)
    D = np.diag(-np.arange(1.0, 11.0) / 3.0)
    announce("f64 diagonal")
    assert q.search_f64(dev_f(D)).triple() == oracle.search_direct_f64(D).triple()


@pytest.mark.parametrize("n,A,k", [(16, 10, 2), (20, 12, 3)])
def test_range_is_subcube_real(q, n, A, k):
    Q = real_matrix(n, 8400 + n)
    Qd = dev_f(Q)
    m_free = n - k
    for m in (0, 1, (1 << k) - 1):
        lo, hi = m << (A - k), (m + 1) << (A - k)
        top = gray(m)
        want = oracle.search_direct_f64(Q, top << m_free, (top + 1) << m_free).triple()
        announce("f64 range", n, A, k, m)
        assert q.search_f64(Qd, prefix_bits=A, gray_lo=lo, gray_hi=hi).triple() == want
        check_coverage(q, n, A, None, lo, hi)


RAGGED_F64 = [(32, 96), (64, 320), (96, 160), (32, 64), (96, 96 + 32 * 9), (160, 1024 + 96),
              (1024 + 32, 2048 - 32), (0, 2048), (224, 544), (256, 480), (480, 1056), (512, 992)]


@pytest.mark.parametrize("lo,hi", RAGGED_F64)
def test_ragged_slices_real(q, lo, hi):
    """Slices that start inside an aligned group of sixteen 32-step bodies (the
    group gate then waits for the next group) or end inside one, or hold one
    whole group between ragged ends, with the exit flips' rows in LDS or in
    global memory; the
    oracle evaluates every state of the slice from the binary64 definition.
    One real matrix (no ties) and one integer-valued (exact sums, many ties)."""
    n, A = 16, 11
    B = n - A
    js = np.arange(lo, hi, dtype=np.uint64)
    pre = (js ^ (js >> np.uint64(1))) << np.uint64(B)
    idx = (pre[:, None] | np.arange(1 << B, dtype=np.uint64)[None, :]).ravel()
    for Q in (real_matrix(n, 8600), np.array(qi.general_uniform(n, 8601, -3, 3), dtype=np.float64)):
        E = oracle.energies_f64(Q, idx)
        m = E.min()
        want = (float(m), int(idx[E == m].min()), int((E == m).sum()))
        Qd = dev_f(Q)
        for cache_bits in (5, 8, 11):
            announce("f64 ragged", lo, hi, cache_bits)
            r = q.search_f64(Qd, prefix_bits=A, cache_bits=cache_bits, gray_lo=lo, gray_hi=hi)
            assert r.triple() == want, (lo, hi, cache_bits)
            check_coverage(q, n, A, None, lo, hi)


@pytest.mark.parametrize("name", ["C1f", "C2f"])
def test_real_configs_vs_stored_oracle(q, name):
    g = golden(name)
    cfg = qi.make_config(name)
    assert qi.sha256_of(cfg["Q"]) == g["sha256_Q"]
    announce("f64 config", name)
    r = q.search_f64(dev_f(cfg["Q"]))
    assert (float.hex(r.min_energy), r.argmin, r.count) == (g["min_energy_hex"], g["argmin"], g["count"])


def test_real_subcubes_at_full_size(q):
    """n = 48 real-valued workload: seeded sub-cubes of 2^28 states against the
    stored oracle results (tests/golden/C4fsub.json), at the default split."""
    g = golden("C4fsub")
    cfg = qi.make_config("C4f")
    assert qi.sha256_of(cfg["Q"]) == g["sha256_Q"]
    A = q.make_plan(48)["prefix_bits"]
    Qd = dev_f(cfg["Q"])
    for cube in g["cubes"]:
        k, top = cube["k"], cube["top"]
        m = inv_gray(top)
        lo, hi = m << (A - k), (m + 1) << (A - k)
        announce("f64 subcube", k, top)
        r = q.search_f64(Qd, prefix_bits=A, gray_lo=lo, gray_hi=hi)
        assert (float.hex(r.min_energy), r.argmin, r.count) == (cube["min_energy_hex"], cube["argmin"],
                                                                 cube["count"]), top


def test_real_full_size_whole_space(q):
    """The whole n = 48 real-valued workload (C4f), checked by what holds at
    any size: the oracle's binary64 energy of the reported minimiser is the
    reported minimum, no single flip of it is lower, and every 32-step body was
    walked once per column group.  And by the oracle on the 2^26-state
    sub-cube that holds the reported minimiser (its first 22 variables fixed):
    the definition's minimum, lowest minimiser and count there are the
    reported ones, and the library's slice search of that sub-cube (the
    benchmark's split, A = 28) returns them too."""
    cfg = qi.make_config("C4f")
    Q = np.asarray(cfg["Q"], dtype=np.float64)
    Qd = dev_f(Q)
    announce("f64 C4f whole space")
    r = q.search_f64(Qd)
    check_coverage(q, 48)
    assert r.count >= 1
    assert oracle.energy_f64(Q, r.argmin) == r.min_energy
    flips = np.asarray([r.argmin ^ (1 << k) for k in range(48)], dtype=np.uint64)
    assert (oracle.energies_f64(Q, flips) >= r.min_energy).all()
    k, free = 22, 26
    top = r.argmin >> free
    announce("f64 C4f oracle on the minimiser's sub-cube", top)
    want = oracle.search_direct_f64(Q, top << free, (top + 1) << free).triple()
    assert want[:2] == (r.min_energy, r.argmin)
    A = q.make_plan(48)["prefix_bits"]
    m = inv_gray(top)
    sub = q.search_f64(Qd, prefix_bits=A, gray_lo=m << (A - k), gray_hi=(m + 1) << (A - k))
    assert sub.triple() == want


def test_integer_valued_full_size(q):
    """The n = 48 integer workload as binary64 gives the integer kernel's triple."""
    import torch
    cfg = qi.make_config("C4")
    Qi = torch.tensor(cfg["Q"], dtype=torch.int32, device="cuda:0")
    announce("C4 int")
    want = q.search(Qi).triple()
    announce("C4 as f64")
    r = q.search_f64(Qi.to(torch.float64))
    assert (r.min_energy, r.argmin, r.count) == (float(want[0]), want[1], want[2])
    check_coverage(q, 48)


def test_concurrent_streams_real(q):
    """Binary64 minimum and spectrum searches and an int32 search, each on a
    stream of its own from its own host thread at the same time, give the
    oracle's answers (each call owns its workspace and timing record)."""
    import threading
    import torch
    Qa, Qb = real_matrix(21, 8601), real_matrix(22, 8602)
    Qi = qi.general_uniform(23, 8603, -50, 50)
    want = [oracle.search_direct_f64(Qa).triple(), oracle.lowest_f64(Qb, 16), oracle.search_gray(Qi).triple()]
    got = [None] * 3
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    if i == 0:
                        got[0] = q.search_f64(dev_f(Qa), stream=s).triple()
                        assert q.last_timing()["states"] == 1 << 21
                    elif i == 1:
                        got[1] = q.lowest(dev_f(Qb), 16, stream=s)
                    else:
                        got[2] = q.search(torch.as_tensor(np.asarray(Qi, dtype=np.int32)).to("cuda:0"),
                                          stream=s).triple()
                        assert q.last_timing()["states"] == 1 << 23
        except Exception as e:  # reported below
            errors.append(e)

    announce("concurrent streams real")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(3)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    assert got == want


def test_f64_errors(q):
    Q = real_matrix(6, 8500)
    for bad in (np.nan, np.inf):
        Qb = Q.copy()
        Qb[2, 3] = bad
        with pytest.raises(q.QuboError) as e:
            q.search_f64(dev_f(Qb))
        assert e.value.code == q.QUBO_ERANGE
    # S below the floor 2^-100 (rejected on the host, before any kernel)
    with pytest.raises(q.QuboError) as e:
        q.search_f64(dev_f(Q * (2.0 ** -100 / np.abs(Q).sum() / 2)))
    assert e.value.code == q.QUBO_ERANGE
    lib = q.load()
    r = q._ResultF64()
    Qd = dev_f(real_matrix(59, 8501))
    assert lib.qubo_search_f64(ctypes.c_void_p(Qd.data_ptr()), 59, -1, -1, 0, 0, 0, None,
                               ctypes.byref(r)) == q.QUBO_EINVAL
    Qd = dev_f(Q)
    assert lib.qubo_search_f64(ctypes.c_void_p(Qd.data_ptr()), 6, -1, -1, 0, 0, q.FLAG_STRICT_MIN, None,
                               ctypes.byref(r)) == q.QUBO_EINVAL
    with pytest.raises(TypeError):
        q.search_f64(Qd.to(dtype=Qd.dtype).float())
