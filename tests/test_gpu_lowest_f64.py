"""Parity of the real-valued (binary64) spectrum, qubo_search_lowest_f64, with
the oracle: the first k states in the order (E ascending, index ascending),
E the binary64 definition summed in row-major order over the set variables.
The bar is bit-exact: the same floats and indices in the same order."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
import qubo_instances as qi
from gpu_helpers import announce, check_coverage, inv_gray

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


def hexpairs(states):
    return [(float.fromhex(e), int(i)) for e, i in states]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 9, 12, 14, 16])
def test_small_real(q, n):
    rng = np.random.default_rng(9500 + n)
    Q = rng.uniform(-10.0, 10.0, size=(n, n))
    Qd = dev_f(Q)
    for k in (1, 7, 64):
        announce("f64 lowest small", n, k)
        assert q.lowest(Qd, k) == oracle.lowest_f64(Q, k), (n, k)


@pytest.mark.parametrize("n,seed,lo,hi", [(6, 9601, -1, 1), (11, 9602, -2, 2), (15, 9603, -1, 1)])
def test_integer_valued_ties(q, n, seed, lo, hi):
    """Integer-valued matrices: exact sums and many equal energies, so the
    index order of ties decides the list; it equals the integer spectrum."""
    Qi = qi.general_uniform(n, seed, lo, hi)
    want = [(float(e), i) for e, i in oracle.lowest(Qi, 64)]
    announce("f64 lowest ties", n, seed)
    assert q.lowest(dev_f(Qi), 64) == want


@pytest.mark.parametrize("n", [5, 14])
def test_every_split(q, n):
    rng = np.random.default_rng(9700 + n)
    Q = np.round(rng.uniform(-4.0, 4.0, size=(n, n)), 1)  # one decimal: inexact sums, some ties
    want = oracle.lowest_f64(Q, 40)
    Qd = dev_f(Q)
    for A in range(5, n + 1):
        for l in sorted({5, (5 + A) // 2, A}):
            announce("f64 lowest split", n, A, l)
            assert q.lowest(Qd, 40, prefix_bits=A, cache_bits=l) == want, (A, l)
            check_coverage(q, n, A, l)


@pytest.mark.parametrize("lo,hi", [(32, 96), (64, 320), (160, 1024 + 96), (0, 2048), (224, 544), (480, 1056)])
def test_ragged_slices(q, lo, hi):
    """Slices that start or end inside an aligned group of sixteen 32-step bodies,
    against the sort of the slice's definition energies."""
    n, A = 16, 11
    B = n - A
    js = np.arange(lo, hi, dtype=np.uint64)
    pre = (js ^ (js >> np.uint64(1))) << np.uint64(B)
    idx = (pre[:, None] | np.arange(1 << B, dtype=np.uint64)[None, :]).ravel()
    Q = np.random.default_rng(9800).uniform(-3.0, 3.0, size=(n, n))
    E = oracle.energies_f64(Q, idx)
    order = np.lexsort((idx, E))[:64]
    want = [(float(E[i]), int(idx[i])) for i in order]
    announce("f64 lowest ragged", lo, hi)
    assert q.lowest(dev_f(Q), 64, prefix_bits=A, gray_lo=lo, gray_hi=hi) == want
    check_coverage(q, n, A, None, lo, hi)


def test_config_vs_stored_oracle(q):
    """The whole real-valued n = 24 workload (C1f): its 64 lowest states."""
    g = golden("C1flow")
    cfg = qi.make_config("C1f")
    assert qi.sha256_of(cfg["Q"]) == g["sha256_Q"]
    announce("f64 lowest C1f")
    assert q.lowest(dev_f(cfg["Q"]), 64) == hexpairs(g["states"])


def test_subcubes_at_full_size(q):
    """The n = 48 real-valued workload at the default split: two seeded
    sub-cubes of 2^28 states against the stored oracle lists, and the integer
    workload as binary64 against the stored integer lists of its sub-cubes."""
    g = golden("C4fsublow")
    cfg = qi.make_config("C4f")
    assert qi.sha256_of(cfg["Q"]) == g["sha256_Q"]
    A = q.make_plan(48)["prefix_bits"]
    Qd = dev_f(cfg["Q"])
    for cube in g["cubes"]:
        k, top = cube["k"], cube["top"]
        m = inv_gray(top)
        lo, hi = m << (A - k), (m + 1) << (A - k)
        announce("f64 lowest subcube", k, top)
        assert q.lowest(Qd, 64, prefix_bits=A, gray_lo=lo, gray_hi=hi) == hexpairs(cube["states"]), top
        check_coverage(q, 48, A, None, lo, hi)
    gi = golden("C4sublow")
    ci = qi.make_config("C4")
    Qi = dev_f(ci["Q"])
    for cube in gi["cubes"][:4]:
        k, top = cube["k"], cube["top"]
        m = inv_gray(top)
        lo, hi = m << (A - k), (m + 1) << (A - k)
        announce("f64 lowest integer subcube", k, top)
        assert q.lowest(Qi, 64, prefix_bits=A, gray_lo=lo, gray_hi=hi) == \
            [(float(e), int(i)) for e, i in cube["states"]], top


def test_whole_space_n48(q):
    """The 64 lowest states of the whole real-valued n = 48 workload, checked by
    what holds at any size: each listed energy is the definition's, the list
    is ordered, it starts with the minimum search's answer, and a single flip of
    a listed state that precedes it in the order is listed too."""
    cfg = qi.make_config("C4f")
    Q = np.asarray(cfg["Q"], dtype=np.float64)
    Qd = dev_f(Q)
    announce("f64 lowest C4f whole space")
    low = q.lowest(Qd, 64)
    check_coverage(q, 48)
    assert len(low) == 64 and low == sorted(low)
    idx = np.asarray([i for _, i in low], dtype=np.uint64)
    assert oracle.energies_f64(Q, idx).tolist() == [e for e, _ in low]
    r = q.search_f64(Qd)
    assert low[0] == (r.min_energy, r.argmin)
    listed = set(low)
    for e, i in low:
        nb = np.asarray([i ^ (1 << b) for b in range(48)], dtype=np.uint64)
        for e2, i2 in zip(oracle.energies_f64(Q, nb).tolist(), nb.tolist()):
            if (e2, i2) < (e, i):
                assert (e2, i2) in listed, ((e, i), (e2, i2))


def test_errors(q):
    Q = np.zeros((6, 6))
    Q[1, 2] = np.nan
    with pytest.raises(q.QuboError) as e:
        q.lowest(dev_f(Q), 4)
    assert e.value.code == q.QUBO_ERANGE
    with pytest.raises(ValueError):
        q.lowest(dev_f(np.zeros((6, 6))), 4, split_bits=1)
