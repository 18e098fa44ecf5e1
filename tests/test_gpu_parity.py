"""Parity of the HIP search (through the C-ABI) with the CPU oracle.

Integer work, so the bar is bit-exact: the same (min_energy, argmin, count) as
the oracle on the same seeded inputs, for every split the library accepts.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
import qubo_instances as qi
from gpu_helpers import announce, check_coverage, dev_q, gray, inv_gray

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


def golden(name):
    path = os.path.join(GOLDEN, name + ".json")
    if not os.path.exists(path):
        pytest.skip("stored oracle result %s.json not written yet" % name)
    with open(path) as f:
        return json.load(f)


# ---------------------------------------------------------------- cache builder

@pytest.mark.parametrize("n,A", [(5, 5), (9, 5), (12, 7), (17, 9), (24, 14), (26, 20), (30, 29), (34, 30),
                                 (32, 32)])
def test_tables_match_definition(q, n, A):
    """E_s, M_int and the Gray-ordered E_p equal energies of states built from
    the definition: E_s[c] = E(c), M_int[v][c] = E(e_v | c) - E(e_v) - E(c),
    EpGray[j] = E(g(j) << B) (eq. 8 of the paper, evaluated by the oracle).
    A = 32 is the largest prefix (24 high bits above the builder's 8 low ones;
    a 16 GiB table, sampled on the device)."""
    import torch
    Q = qi.general_uniform(n, 5000 + n, -100, 100)
    B = n - A
    announce("tables", n, A)
    es, mint, ep_dev = q.build_tables(dev_q(Q), A)
    es, mint = es.cpu().numpy(), mint.cpu().numpy()
    cols = np.arange(1 << B, dtype=np.uint64)
    if cols.size > 4096:
        cols = np.unique(np.concatenate([cols[:1024], cols[-1024:],
                                         np.random.default_rng(n).choice(cols, 2048)]))
    Ec = oracle.energies(Q, cols)
    assert np.array_equal(es[cols.astype(np.int64)], Ec)
    for v in range(A):
        ev = np.uint64(1 << (n - 1 - v))
        want = oracle.energies(Q, cols | ev) - Ec - oracle.energy(Q, int(ev))
        assert np.array_equal(mint[v, cols.astype(np.int64)], want), v
    if A <= 13:
        js = np.arange(1 << A, dtype=np.uint64)
    else:  # both ends and a seeded sample, drawn without listing all 2^A steps
        js = np.unique(np.concatenate([np.arange(2048, dtype=np.uint64),
                                       np.arange((1 << A) - 2048, 1 << A, dtype=np.uint64),
                                       np.random.default_rng(A).integers(0, 1 << A, 4096, dtype=np.uint64)]))
    states = (js ^ (js >> np.uint64(1))) << np.uint64(B)
    ep = ep_dev[torch.as_tensor(js.astype(np.int64), device=ep_dev.device)].cpu().numpy()
    del ep_dev
    torch.cuda.synchronize()
    assert np.array_equal(ep, oracle.energies(Q, states))


# ---------------------------------------------------------------- small instances

SMALL = [(n, 6000 + n, -100, 100) for n in range(1, 21)] + \
        [(n, 6100 + n, -2, 2) for n in (5, 9, 14, 18)] + \
        [(n, 6200 + n, -1, 1) for n in (6, 11, 16)]


@pytest.mark.parametrize("n,seed,lo,hi", SMALL)
def test_small_random(q, n, seed, lo, hi):
    """Non-symmetric Q, with and without heavy ties, against oracle tier B, in
    both kernel modes (bound-gated default and strict per-step minimum)."""
    Q = qi.general_uniform(n, seed, lo, hi)
    want = oracle.search_gray(Q).triple()
    Qd = dev_q(Q)
    for R in (8, 16):
        for strict in (False, True):
            announce("small", n, seed, lo, hi, R, "strict" if strict else "gated")
            assert q.search(Qd, strict=strict, cols_per_lane=R).triple() == want, (R, strict)
            check_coverage(q, n, strict=strict, cols_per_lane=R)


@pytest.mark.parametrize("n", [5, 11, 18, 22])
def test_every_split(q, n):
    """The result does not depend on the prefix/suffix split or the cache size
    (permutation invariance, sec. II.D): every accepted split is exact."""
    Q = qi.general_uniform(n, 6300 + n, -50, 50)
    want = oracle.search_gray(Q).triple()
    Qd = dev_q(Q)
    for A in range(5, n + 1):
        for l in sorted({5, min(A, 7), min(A, 13), A} & set(range(5, min(A, 21) + 1))):
            for strict, R in ((False, 8), (True, 8), (False, 16), (True, 16)):
                announce("split", n, A, l, strict, R)
                got = q.search(Qd, prefix_bits=A, cache_bits=l, strict=strict, cols_per_lane=R)
                assert got.triple() == want, (A, l, strict, R)
                check_coverage(q, n, A, l, strict=strict, cols_per_lane=R)


@pytest.mark.parametrize("strict", [False, True])
def test_special_cases(q, strict):
    for n in (3, 7, 16, 21):
        zero = qi.zeros(n)
        announce("zero", n)
        assert q.search(dev_q(zero), strict=strict).triple() == (0, 0, 1 << n)
        diag = qi.zeros(n)
        for i in range(n):
            diag[i][i] = -(i + 1)
        announce("negative diagonal", n)
        assert q.search(dev_q(diag), strict=strict).triple() == (-n * (n + 1) // 2, (1 << n) - 1, 1)
        for i in range(n):
            diag[i][i] = i + 1
        announce("positive diagonal", n)
        assert q.search(dev_q(diag), strict=strict).triple() == (0, 0, 1)


def test_planted_and_mattis(q):
    for n, seed in [(9, 7001), (23, 7002), (30, 7003)]:
        Q, P, a = qi.planted(n, seed)
        av = np.asarray(a, dtype=np.int64)
        want = (-int(av @ np.asarray(P, dtype=np.int64) @ av), qi.bits_to_index(a), 1)
        announce("planted", n, seed)
        assert q.search(dev_q(Q)).triple() == want
    for n, seed in [(6, 7101), (25, 7102), (33, 7103)]:
        J, h, xi = qi.mattis(n, seed)
        Q, C = qi.ising_to_qubo(J, h)
        xa = [(1 + s) // 2 for s in xi]
        want_arg = min(qi.bits_to_index(xa), qi.bits_to_index([1 - v for v in xa]))
        announce("mattis", n, seed)
        r = q.search(dev_q(Q))
        assert (r.min_energy + C, r.argmin, r.count) == (-n * (n - 1) // 2, want_arg, 2)


def test_extreme_entries(q):
    """Entries near the overflow guard: sum |Q_ij| just under 2^30."""
    n = 12
    big = (2 ** 30 - 1) // (n * n)
    Q = qi.general_uniform(n, 7201, -big, big)
    want = oracle.search_gray(Q).triple()
    announce("extreme", n, big)
    assert q.search(dev_q(Q)).triple() == want
    assert q.search(dev_q(Q), prefix_bits=6, cache_bits=6).triple() == want


@pytest.mark.parametrize("sign", [-1, 1])
def test_extreme_one_signed(q, sign):
    """Near the overflow guard with every entry of one sign: the search's table
    offsets (each row and the suffix energies raised by the sum of their
    negative parts) are then as large as the entries allow (all negative) or
    zero (all positive).  Padding columns (2^5 columns in a group of 512) and
    the pair and group gates at several splits, with the strict per-step
    minimum and 16 columns per lane; the minimum and the 8 lowest."""
    n = 12
    big = (2 ** 30 - 1) // (n * n)
    Q = [[sign * abs(v) for v in row] for row in qi.general_uniform(n, 7202, -big, big)]
    want = oracle.search_gray(Q).triple()
    low = oracle.lowest(Q, 8)
    Qd = dev_q(Q)
    for A in (None, 6, 7, 9):
        for strict, R in ((False, 8), (True, 8), (False, 16)):
            announce("extreme one-signed", sign, A, strict, R)
            assert q.search(Qd, prefix_bits=A, strict=strict, cols_per_lane=R).triple() == want, (A, strict, R)
        assert q.lowest(Qd, 8, prefix_bits=A) == low, A


# ---------------------------------------------------------------- configs

@pytest.mark.parametrize("name,splits", [
    ("C1", [(None, None), (14, 5), (19, 13), (10, 10), (24, 20)]),
    ("C2", [(None, None), (22, 13), (16, 9), (26, 18)]),
    ("C2p", [(None, None), (20, 12)]),
    ("C3", [(None, None), (28, 13), (30, 16), (26, 8)]),
])
def test_config_vs_stored_oracle(q, name, splits):
    g = golden(name)
    cfg = qi.make_config(name)
    assert qi.sha256_of(cfg["Q"]) == g["sha256_Q"]
    want = (g["min_energy"], g["argmin"], g["count"])
    Qd = dev_q(cfg["Q"])
    for A, l in splits:
        for strict, R in ((False, 8), (True, 8), (False, 16), (True, 16)):
            announce("config", name, A, l, strict, R)
            got = q.search(Qd, prefix_bits=A, cache_bits=l, strict=strict, cols_per_lane=R)
            assert got.triple() == want, (A, l, strict, R)
            check_coverage(q, cfg["n"], A, l, strict=strict, cols_per_lane=R)


# ---------------------------------------------------------------- slices

@pytest.mark.parametrize("n,A,k", [(20, 12, 3), (24, 14, 6), (28, 20, 4)])
def test_range_is_subcube(q, n, A, k):
    """The Gray range [m 2^(A-k), (m+1) 2^(A-k)) is the sub-cube whose first k
    variables spell g(m) (sec. III.C.1); compare with oracle tier B on it."""
    Q = qi.general_uniform(n, 7300 + n, -100, 100)
    for m in (0, 1, (1 << k) - 1, (1 << k) // 3):
        lo, hi = m << (A - k), (m + 1) << (A - k)
        want = oracle.search_gray(Q, k=k, top=gray(m)).triple()
        for strict, R in ((False, 8), (True, 8), (False, 16), (True, 16)):
            announce("range", n, A, k, m, strict, R)
            assert q.search_range(dev_q(Q), A, lo, hi, strict=strict, cols_per_lane=R).triple() == want
            check_coverage(q, n, A, None, lo, hi, strict=strict, cols_per_lane=R)


# (96, 288): bodies 3..8, an aligned quarter of a group between ragged ends;
# (128, 224): bodies 4..6; (256, 512) bodies 8..15; (224, 544) bodies 7..16;
# (256, 480) bodies 8..14; (640, 1152) bodies 20..35.  The group gate covers
# aligned groups of sixteen bodies: (512, 1024) is bodies 16..31, one whole
# group; (480, 1056) bodies 15..32, a whole group between ragged ends;
# (512, 992) bodies 16..30, a group start without its sixteenth body.
RAGGED = [(32, 96), (96, 160), (0, 32), (32, 64), (64, 128 + 32), (1024 + 32, 2048 - 32), (0, 2048),
          (96, 288), (128, 224), (256, 512), (224, 544), (256, 480), (640, 1152), (512, 1024), (480, 1056),
          (512, 992)]


def _slice_states(n, A, lo, hi):
    """Indices of the states the slice [lo, hi) of the Gray walk covers."""
    B = n - A
    js = np.arange(lo, hi, dtype=np.uint64)
    pre = (js ^ (js >> np.uint64(1))) << np.uint64(B)
    return (pre[:, None] | np.arange(1 << B, dtype=np.uint64)[None, :]).ravel()


@pytest.mark.parametrize("lo,hi", RAGGED)
def test_ragged_slices(q, lo, hi):
    """Slices that start or end on an odd 32-step body (or hold one body), so
    that the 128-step group bound, the 64-step pair bound and the single-body
    bound all decide; the oracle evaluates every state of the slice from the
    definition."""
    n, A = 16, 11
    Q = qi.general_uniform(n, 7350, -4, 4)
    idx = _slice_states(n, A, lo, hi)
    E = oracle.energies(Q, idx)
    m = int(E.min())
    want = (m, int(idx[E == m].min()), int((E == m).sum()))
    Qd = dev_q(Q)
    for strict, R in ((False, 8), (True, 8), (False, 16)):
        announce("ragged", lo, hi, strict, R)
        assert q.search_range(Qd, A, lo, hi, strict=strict, cols_per_lane=R).triple() == want
        check_coverage(q, n, A, None, lo, hi, strict=strict, cols_per_lane=R)
    order = np.lexsort((idx, E))[:64]
    announce("ragged lowest", lo, hi)
    assert q.lowest(Qd, 64, prefix_bits=A, gray_lo=lo, gray_hi=hi) == \
        [(int(E[i]), int(idx[i])) for i in order]


def _aligned_blocks(lo, hi):
    """[lo, hi) as maximal aligned blocks [m 2^s, (m + 1) 2^s): (m, s) pairs.
    Each block of Gray steps is the sub-cube whose first A - s variables spell
    g(m) (sec. III.C.1)."""
    while lo < hi:
        s = (lo & -lo).bit_length() - 1 if lo else (hi - lo).bit_length()
        while (1 << s) > hi - lo:
            s -= 1
        yield lo >> s, s
        lo += 1 << s


def _combine(triples):
    """min; count at the min; lowest index at the min (the final reduction's rule)."""
    m = min(t[0] for t in triples)
    return (m, min(t[1] for t in triples if t[0] == m), sum(t[2] for t in triples if t[0] == m))


# Slices of about 40 segments of 2^10 Gray steps, so that the number of segment
# blocks (four segments each) is not a power of two and the work-item order has
# empty slots, over 2 (n = 26) and 8 (n = 30) column groups of 512 columns.
TILE_SLICES = [(26, 16, 3 * 1024 + 96, 41 * 1024 + 160), (30, 18, 5 * 1024 + 32, 52 * 1024 + 64)]


@pytest.mark.parametrize("n,A,lo,hi", TILE_SLICES)
def test_slices_across_tiles(q, n, A, lo, hi):
    """Minimum, lowest minimiser and count of a ragged slice against oracle tier
    B on its aligned sub-cubes, gated and strict, 8 and 16 columns per lane; the
    16 lowest states against the oracle's lists of the same sub-cubes."""
    Q = qi.general_uniform(n, 7400 + n, -100, 100)
    blocks = list(_aligned_blocks(lo, hi))
    assert sum(1 << s for _, s in blocks) == hi - lo
    want = _combine([oracle.search_gray(Q, k=A - s, top=gray(m)).triple() for m, s in blocks])
    plan = q.make_plan(n, A)
    assert plan["seg_bits"] == 10, plan  # segments of 2^10 steps: 39 and 48 segments
    Qd = dev_q(Q)
    for strict, R in ((False, 8), (True, 8), (False, 16), (True, 16)):
        announce("slice across tiles", n, A, lo, hi, strict, R)
        assert q.search_range(Qd, A, lo, hi, strict=strict, cols_per_lane=R).triple() == want
        check_coverage(q, n, A, None, lo, hi, strict=strict, cols_per_lane=R)
    lists = []
    for m, s in blocks:
        lists += oracle.lowest(Q, 16, fixed=A - s, top=gray(m))
    announce("slice across tiles, 16 lowest", n, A, lo, hi)
    assert q.lowest(Qd, 16, prefix_bits=A, gray_lo=lo, gray_hi=hi) == sorted(lists)[:16]


def test_f64_slice_across_tiles(q):
    """The binary64 search of a ragged slice over several segment blocks
    (2^10-step segments, 39 of them) against the binary64 oracle on the index
    ranges of its aligned sub-cubes."""
    import torch
    n, A, lo, hi = 22, 16, 3 * 1024 + 96, 41 * 1024 + 160
    Q = qi.general_uniform_f64(n, 7450, -10.0, 10.0)
    B = n - A
    parts = []
    for m, s in _aligned_blocks(lo, hi):
        top = gray(m)  # the first A - s variables
        base = top << (B + s)
        r = oracle.search_direct_f64(Q, lo=base, hi=base + (1 << (B + s)))
        parts.append(r.triple())
    want = _combine(parts)
    announce("f64 slice across tiles", n, A, lo, hi)
    got = q.search_f64(torch.tensor(Q, dtype=torch.float64, device="cuda:0"), prefix_bits=A,
                       gray_lo=lo, gray_hi=hi).triple()
    assert got == want, (got, want)


@pytest.mark.parametrize("name", ["C4sub", "C5sub", "C4sub36", "C5sub37"])
def test_subcubes_at_full_size(q, name):
    """n = 48 and n = 50 at the benchmark's split (A = 28): seeded sub-cubes
    against the stored oracle results, each in one of the four kernel builds
    (bound-gated or strict, 8 or 16 columns per lane).  C4sub and C5sub hold
    2^32 states (2^12 and 2^10 Gray steps); C4sub36 and C5sub37 hold 2^36 and
    2^37 states (2^16 and 2^15 Gray steps), so the walk flips prefix bits at
    and above cache_bits, whose rows come from global memory."""
    g = golden(name)
    cfg = qi.make_config(name[:2])
    assert qi.sha256_of(cfg["Q"]) == g["sha256_Q"]
    n = cfg["n"]
    plan = q.make_plan(n)
    A = plan["prefix_bits"]
    Qd = dev_q(cfg["Q"])
    for i, cube in enumerate(g["cubes"]):
        k, top = cube["k"], cube["top"]
        m = inv_gray(top)
        lo, hi = m << (A - k), (m + 1) << (A - k)
        if name.endswith(("36", "37")):
            assert (hi - lo) >> plan["cache_bits"] >= 2  # bits above the cached ones flip
        strict, R = bool(i % 2), (8 if i % 4 < 2 else 16)
        announce("subcube", name, k, top, strict, R)
        r = q.search_range(Qd, A, lo, hi, strict=strict, cols_per_lane=R)
        assert r.triple() == (cube["min_energy"], cube["argmin"], cube["count"])
        check_coverage(q, n, A, None, lo, hi, strict=strict, cols_per_lane=R)


def test_long_slice_at_full_size(q):
    """n = 48 at the benchmark's split: a slice of 2^20 Gray steps (2^40 states)
    that starts in the middle of a 2^18-step work-unit segment, so it spans five
    segments (a part of the first, three whole, a part of the last) and every
    wave of a workgroup walks one; against the stored oracle result
    (tests/golden/C4slice.json: eight consecutive sub-cubes, combined by the
    final reduction's rule), in all four kernel builds, and per sub-cube."""
    g = golden("C4slice")
    cfg = qi.make_config("C4")
    assert qi.sha256_of(cfg["Q"]) == g["sha256_Q"]
    n = cfg["n"]
    plan = q.make_plan(n)
    A, seg = plan["prefix_bits"], plan["seg_bits"]
    k, j0, c = g["k"], g["j_first"], g["cubes_in_slice"]
    assert [cube["top"] for cube in g["cubes"]] == [gray(j) for j in range(j0, j0 + c)]
    lo, hi = j0 << (A - k), (j0 + c) << (A - k)
    assert lo % (1 << seg) != 0 and (hi - 1 >> seg) - (lo >> seg) + 1 >= 5
    Qd = dev_q(cfg["Q"])
    for strict, R in ((False, 8), (True, 8), (False, 16), (True, 16)):
        announce("long slice", lo, hi, strict, R)
        r = q.search_range(Qd, A, lo, hi, strict=strict, cols_per_lane=R)
        assert r.triple() == (g["min_energy"], g["argmin"], g["count"]), (strict, R)
        check_coverage(q, n, A, None, lo, hi, strict=strict, cols_per_lane=R)
    for cube in g["cubes"]:
        j = cube["j"]
        announce("long slice cube", j)
        r = q.search_range(Qd, A, j << (A - k), (j + 1) << (A - k))
        assert r.triple() == (cube["min_energy"], cube["argmin"], cube["count"]), j


@pytest.mark.parametrize("n,k,seed,lo,hi", [(9, 4, 7501, -50, 50), (14, 3, 7502, -2, 2),
                                            (20, 6, 7503, -100, 100), (26, 2, 7504, -1, 1)])
def test_outer_split(q, n, k, seed, lo, hi):
    """Fixing the first k variables and searching the 2^k reduced sub-problems
    (sec. III.C.1, used automatically above 58 variables) gives the oracle's
    answer, ties included; later sub-problems are capped by the best so far."""
    Q = qi.general_uniform(n, seed, lo, hi)
    want = oracle.search_gray(Q).triple()
    Qd = dev_q(Q)
    for strict in (False, True):
        announce("split", n, k, seed, strict)
        assert q.search(Qd, split_bits=k, strict=strict).triple() == want, (k, strict)
    t = q.last_timing()
    assert t["states"] <= 1 << n
    with pytest.raises(q.QuboError):
        q.search(Qd, split_bits=n - 4)


def test_deterministic(q):
    Q = qi.make_config("C2")["Q"]
    Qd = dev_q(Q)
    announce("determinism C2")
    first = q.search(Qd).triple()
    for _ in range(3):
        assert q.search(Qd).triple() == first


def test_errors(q):
    Qd = dev_q(qi.general_uniform(10, 7400, -5, 5))
    with pytest.raises(q.QuboError) as e:
        q.search(Qd, prefix_bits=3)
    assert e.value.code == q.QUBO_EPLAN
    with pytest.raises(q.QuboError) as e:
        q.search(Qd, prefix_bits=11)
    assert e.value.code == q.QUBO_EINVAL
    with pytest.raises(q.QuboError) as e:
        q.search(Qd, prefix_bits=8, cache_bits=9)
    assert e.value.code == q.QUBO_EINVAL
    with pytest.raises(q.QuboError) as e:
        q.search_range(Qd, 8, 0, 33)
    assert e.value.code == q.QUBO_EINVAL
    big = dev_q([[2 ** 30, 0], [0, 0]])
    with pytest.raises(q.QuboError) as e:
        q.search(big)
    assert e.value.code == q.QUBO_ERANGE


def test_concurrent_streams(q):
    """Calls on different streams from different host threads run concurrently
    (each call owns its workspace and timing record) and give the same answers
    as alone."""
    import threading
    import torch
    cases = [qi.general_uniform(n, 7600 + n, -50, 50) for n in (22, 23, 24, 25)]
    want = [oracle.search_gray(Q).triple() for Q in cases]
    got = [None] * len(cases)
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                Qd = dev_q(cases[i])
                for _ in range(3):
                    got[i] = q.search(Qd, stream=s).triple()
                    assert q.last_timing()["states"] == 1 << len(cases[i])
        except Exception as e:  # reported below
            errors.append(e)

    announce("concurrent streams")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    assert got == want
