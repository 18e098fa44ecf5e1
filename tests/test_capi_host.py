"""Host-side checks of the C-ABI library (no GPU needed).

The library must load on a machine without a GPU and export every symbol
include/qubo.h declares; planning, the overflow guard and argument validation
run on the host only.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import ising_ground_state_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    with open(os.path.join(ROOT, "include", "qubo.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"QUBO_API\s+[\w\s\*]*?\b(qubo_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = q.load()
    names = declared_symbols()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(q.EXPORTS)


def test_version_and_strerror():
    assert "gfx950" in q.version()
    for code in (0, -1, -2, -3, -4, -5, -6, -99):
        assert q.strerror(code)


@pytest.mark.parametrize("n", [1, 2, 4, 5, 6, 12, 24, 32, 40, 48, 50, 56, 58, 59, 63])
def test_plan_invariants(n):
    p = q.make_plan(n)
    k = p["split_bits"]
    assert k == max(0, n - 58)
    assert p["n"] == n and p["n_search"] == max(n - k, 5)
    A, B = p["prefix_bits"], p["suffix_bits"]
    assert A + B == p["n_search"] and A >= 5 and A <= 32
    assert 5 <= p["cache_bits"] <= A
    assert 5 <= p["seg_bits"] <= min(A, 18)
    group = 64 * p["cols_per_lane"]
    assert p["cols_per_lane"] in (8, 16)
    assert p["lds_bytes"] == max(0, min(p["cache_bits"], p["seg_bits"]) - 5) * group * 4 <= 65536
    assert p["col_groups"] == max(1, (1 << B) // group)
    assert p["work_units"] == p["col_groups"] << (A - p["seg_bits"])
    # the whole space is covered: units x steps x columns per group >= 2^n per sub-problem
    assert p["work_units"] * (1 << p["seg_bits"]) * group >= 1 << p["n_search"]
    assert p["workspace_bytes"] >= 4 * ((1 << A) + A * max(1 << B, group))


def test_plan_explicit_splits():
    p = q.make_plan(48, prefix_bits=28, cache_bits=16)
    assert (p["prefix_bits"], p["suffix_bits"], p["cache_bits"]) == (28, 20, 16)
    assert p["lds_bytes"] == 11 * 64 * p["cols_per_lane"] * 4
    p = q.make_plan(48, prefix_bits=28, cache_bits=5)
    assert p["lds_bytes"] == 0
    # cached bits beyond one work unit's segment never flip there: the plan reports the effective value
    p = q.make_plan(40, prefix_bits=30, cache_bits=22)
    assert p["cache_bits"] == p["seg_bits"] <= 18


@pytest.mark.parametrize("args,code", [
    ((0, -1, -1), q.QUBO_EINVAL), ((64, -1, -1), q.QUBO_EINVAL),
    ((10, 11, -1), q.QUBO_EINVAL), ((10, 8, 9), q.QUBO_EINVAL), ((10, -2, -1), q.QUBO_EINVAL),
    ((10, 4, -1), q.QUBO_EPLAN), ((10, 8, 4), q.QUBO_EPLAN),
    ((40, 33, -1), q.QUBO_EPLAN),
])
def test_plan_rejects(args, code):
    with pytest.raises(q.QuboError) as e:
        q.make_plan(*args)
    assert e.value.code == code


def test_check_q_guard():
    Q = np.zeros((3, 3), dtype=np.int32)
    Q[0, 1] = 2 ** 29
    Q[2, 0] = -(2 ** 29 - 1)
    assert q.check_q(Q) == 2 ** 30 - 1
    Q[1, 1] = 1
    with pytest.raises(q.QuboError) as e:
        q.check_q(Q)
    assert e.value.code == q.QUBO_ERANGE
    R = np.asarray([[3, -5], [1, 2]], dtype=np.int32)
    assert q.check_q(R) == 11


def test_check_q_f64_guard():
    """The binary64 guard: finite entries and S = sum |Q_ij| either 0 or in
    [2^-100, 2^100].  The range keeps the walk's scale factor 2^(17 - e)
    (S < 2^e) and the binary64 sums well inside binary64's normal range."""
    q.check_q_f64(np.zeros((4, 4)))
    q.check_q_f64(-np.zeros((4, 4)))  # negative zeros: S = 0
    for bad in (np.nan, np.inf, -np.inf):
        Q = np.ones((3, 3))
        Q[1, 2] = bad
        with pytest.raises(q.QuboError) as e:
            q.check_q_f64(Q)
        assert e.value.code == q.QUBO_ERANGE
    # S just above the floor passes, just below it fails; the sum is rounded up
    # by the guard (a factor 1 + 2^-40), so test a little way from 2^-100
    Q = np.zeros((2, 2))
    Q[0, 0] = 2.0 ** -100 * (1 + 2.0 ** -30)
    q.check_q_f64(Q)
    Q[0, 0] = 2.0 ** -100 * (1 - 2.0 ** -30)
    with pytest.raises(q.QuboError) as e:
        q.check_q_f64(Q)
    assert e.value.code == q.QUBO_ERANGE
    # entries 2^-40 below the floor next to one that lifts S above it
    Q = np.full((3, 3), 2.0 ** -140)
    Q[2, 2] = 2.0 ** -99
    q.check_q_f64(Q)
    Q[2, 2] = 2.0 ** -102
    with pytest.raises(q.QuboError) as e:
        q.check_q_f64(Q)
    assert e.value.code == q.QUBO_ERANGE
    # the upper end
    Q = np.zeros((2, 2))
    Q[0, 1] = 2.0 ** 99
    q.check_q_f64(Q)
    Q[1, 0] = 2.0 ** 99 * 1.01
    with pytest.raises(q.QuboError) as e:
        q.check_q_f64(Q)
    assert e.value.code == q.QUBO_ERANGE


def test_f64_as_int32():
    """The int32 form of a dyadic binary64 matrix (the binary64 searches' integer
    path): the smallest exponent f, Q = Q_int / 2^f entry by entry, the limit
    sum |Q_int| <= 2^30 - 1, and refusal of everything else."""
    import oracle
    import qubo_instances as qi
    Qi = np.array(qi.general_uniform(10, 8951, -5, 5), dtype=np.int64)
    assert (Qi % 2 != 0).any()
    Qint, f = q.f64_as_int32(Qi.astype(np.float64))
    assert f == 0 and (Qint == Qi).all()
    Qint, f = q.f64_as_int32(Qi / 8.0)
    assert f == 3 and (Qint == Qi).all()
    Qint, f = q.f64_as_int32(Qi * 2.0 ** 40)  # multiples of 2^40: f < 0
    assert f == -40 and (Qint == Qi).all()
    Qint, f = q.f64_as_int32(np.zeros((3, 3)))
    assert f == 0 and not Qint.any()
    Qint, f = q.f64_as_int32(-np.zeros((3, 3)))
    assert f == 0 and not Qint.any()
    # the limit: sum |2^f Q| = 2^30 - 1 passes, 2^30 + 1 fails (f = 0: odd entries)
    Q = np.zeros((2, 2))
    Q[0, 0], Q[1, 1] = 2.0 ** 29, -(2.0 ** 29 - 1)
    assert q.f64_as_int32(Q)[1] == 0
    Q[1, 1] = -(2.0 ** 29 + 1)
    with pytest.raises(q.QuboError) as e:
        q.f64_as_int32(Q)
    assert e.value.code == q.QUBO_ERANGE
    Q[1, 1] = -(2.0 ** 29 - 1)
    assert q.f64_as_int32(Q / 2.0 ** 10)[1] == 10  # the same limit after scaling
    for bad in (0.1, np.pi, 2.0 ** -1074, np.nan, np.inf):
        Q = np.ones((3, 3))
        Q[0, 1] = bad
        with pytest.raises(q.QuboError) as e:
            q.f64_as_int32(Q)
        assert e.value.code == q.QUBO_ERANGE, bad
    Q = np.ones((3, 3))
    Q[2, 2] = 2.0 ** -30  # dyadic, but 2^30 sum |Q| is above the limit
    with pytest.raises(q.QuboError):
        q.f64_as_int32(Q)
    # the point of the form: the binary64 definition's energy of every state is
    # E_int / 2^f exactly (oracle tier A in binary64 and in int64)
    Q = Qi / 8.0
    Qint, f = q.f64_as_int32(Q)
    idx = np.arange(1 << 10, dtype=np.uint64)
    assert (oracle.energies_f64(Q, idx) == oracle.energies(Qint, idx) / 2.0 ** f).all()


def test_null_and_range_arguments_rejected_before_the_device():
    lib = q.load()
    r = q._Result()
    assert lib.qubo_search(None, 10, -1, -1, None, ctypes.byref(r)) == q.QUBO_EINVAL
    assert lib.qubo_search(ctypes.c_void_p(16), 0, -1, -1, None, ctypes.byref(r)) == q.QUBO_EINVAL
    assert lib.qubo_search(ctypes.c_void_p(16), 64, -1, -1, None, ctypes.byref(r)) == q.QUBO_EINVAL
    assert lib.qubo_search(ctypes.c_void_p(16), 10, -1, -1, None, None) == q.QUBO_EINVAL
    # slices must be 32-aligned, non-empty and inside the prefix walk
    for lo, hi in [(0, 33), (1, 64), (64, 64), (0, 1 << 9), (32, 0)]:
        assert lib.qubo_search_range(ctypes.c_void_p(16), 12, 8, -1, lo, hi, None,
                                     ctypes.byref(r)) == q.QUBO_EINVAL
    assert lib.qubo_search_range(ctypes.c_void_p(16), 4, 4, -1, 0, 32, None,
                                 ctypes.byref(r)) == q.QUBO_EINVAL
    assert lib.qubo_build_tables(ctypes.c_void_p(16), 12, 6, None, None, None, None) == q.QUBO_EINVAL
    assert lib.qubo_check_q(None, 3) == q.QUBO_EINVAL
    assert lib.qubo_check_q_f64(None, 3) == q.QUBO_EINVAL
    s = ctypes.c_int64(-7)
    assert lib.qubo_abs_sum(None, 3, ctypes.byref(s)) == q.QUBO_EINVAL
    z = np.zeros((3, 3), dtype=np.int32)
    assert lib.qubo_abs_sum(z.ctypes.data_as(ctypes.c_void_p), 3, None) == q.QUBO_EINVAL
    assert lib.qubo_abs_sum(z.ctypes.data_as(ctypes.c_void_p), 64, ctypes.byref(s)) == q.QUBO_EINVAL
    assert s.value == -7
    assert r.count == 0  # untouched
    # spectrum: k in 1..64, outputs present, no strict mode, no unknown flags, valid slices
    out = (q._State * 64)()
    found = ctypes.c_int(-3)
    P = ctypes.c_void_p(16)
    for k, flags, lo, hi, o, fo in [(0, 0, 0, 0, out, found), (65, 0, 0, 0, out, found),
                                    (4, q.FLAG_STRICT_MIN, 0, 0, out, found), (4, 1 << 20, 0, 0, out, found),
                                    (4, q.FLAG_COLS8 | q.FLAG_COLS16, 0, 0, out, found),
                                    (4, 0, 0, 33, out, found), (4, 0, 0, 0, None, found),
                                    (4, 0, 0, 0, out, None)]:
        fp = ctypes.byref(fo) if fo is not None else None
        assert lib.qubo_search_lowest(P, 12, k, 8, -1, lo, hi, flags, None, o, fp) == q.QUBO_EINVAL, (k, flags)
    assert lib.qubo_search_lowest(None, 12, 4, -1, -1, 0, 0, 0, None, out, ctypes.byref(found)) == q.QUBO_EINVAL
    assert found.value == -3  # untouched
    # real-valued search: n in 1..58 (no outer split), only the 8-column flag, valid slices
    rf = q._ResultF64()
    for n_, flags, lo, hi in [(0, 0, 0, 0), (59, 0, 0, 0), (12, q.FLAG_STRICT_MIN, 0, 0),
                              (12, q.FLAG_COLS16, 0, 0), (12, 0, 0, 33)]:
        assert lib.qubo_search_f64(P, n_, 8, -1, lo, hi, flags, None, ctypes.byref(rf)) == q.QUBO_EINVAL, n_
    assert lib.qubo_search_f64(None, 12, -1, -1, 0, 0, 0, None, ctypes.byref(rf)) == q.QUBO_EINVAL
    assert lib.qubo_search_f64(P, 12, -1, -1, 0, 0, 0, None, None) == q.QUBO_EINVAL
    # real-valued spectrum: k in 1..64, outputs present, n in 1..58, the 8-column flag only, valid slices
    outf = (q._StateF64 * 64)()
    foundf = ctypes.c_int(-7)
    for n_, k, flags, lo, hi, o, fo in [(12, 0, 0, 0, 0, outf, foundf), (12, 65, 0, 0, 0, outf, foundf),
                                        (59, 4, 0, 0, 0, outf, foundf), (0, 4, 0, 0, 0, outf, foundf),
                                        (12, 4, q.FLAG_COLS16, 0, 0, outf, foundf),
                                        (12, 4, q.FLAG_STRICT_MIN, 0, 0, outf, foundf),
                                        (12, 4, 0, 0, 33, outf, foundf), (12, 4, 0, 0, 0, None, foundf),
                                        (12, 4, 0, 0, 0, outf, None)]:
        fp = ctypes.byref(fo) if fo is not None else None
        assert lib.qubo_search_lowest_f64(P, n_, k, 8, -1, lo, hi, flags, None, o, fp) == q.QUBO_EINVAL, \
            (n_, k, flags, lo, hi)
    assert lib.qubo_search_lowest_f64(None, 12, 4, -1, -1, 0, 0, 0, None, outf, ctypes.byref(foundf)) == \
        q.QUBO_EINVAL
    assert foundf.value == -7  # untouched


def test_progress_record_and_rejections_before_the_device():
    """The run state of a search in slices is a fixed 96-byte record; malformed
    arguments and records are refused before any device call, and a finished
    run's step does nothing."""
    lib = q.load()
    assert ctypes.sizeof(q.Progress) == 96
    offsets = {name: getattr(q.Progress, name).offset for name, _ in q.Progress._fields_}
    assert offsets == {"q_hash": 0, "n": 8, "split_bits": 12, "prefix_bits": 16, "chunk_bits": 20,
                       "sub": 24, "next": 32, "steps_done": 40, "steps_total": 48, "done": 56,
                       "have_best": 60, "u": 64, "kind": 88, "reserved": 92}
    assert q.Progress.best.offset == q.Progress.best_f64.offset == 64
    P = ctypes.c_void_p(16)
    p = q.Progress()
    assert lib.qubo_progress_init(None, 12, -1, -1, 0, None, ctypes.byref(p)) == q.QUBO_EINVAL
    assert lib.qubo_progress_init(P, 12, -1, -1, 0, None, None) == q.QUBO_EINVAL
    for n_, pb, cb, flags in [(0, -1, -1, 0), (64, -1, -1, 0), (12, -1, -1, q.FLAG_STRICT_MIN),
                              (12, -1, -1, q.FLAG_COLS8), (12, 8, 4, 0), (12, 8, 9, 0),
                              (12, -1, -1, 8 << q.FLAG_SPLIT_SHIFT)]:
        assert lib.qubo_progress_init(P, n_, pb, cb, flags, None, ctypes.byref(p)) == q.QUBO_EINVAL, (n_, pb, cb)
    assert bytes(p) == bytes(96)  # untouched
    # a record that does not describe a run of this n, or is out of range
    good = dict(n=12, split_bits=0, prefix_bits=8, chunk_bits=6, steps_total=4)
    bad = [dict(n=13), dict(split_bits=-1), dict(split_bits=8), dict(prefix_bits=4), dict(prefix_bits=13),
           dict(chunk_bits=4), dict(chunk_bits=9), dict(next=32), dict(next=1 << 8), dict(sub=1),
           dict(steps_total=0)]
    for change in bad:
        p = q.Progress(**{**good, **change})
        before = bytes(p)
        assert lib.qubo_search_step(P, 12, None, ctypes.byref(p)) == q.QUBO_EINVAL, change
        assert bytes(p) == before
    assert lib.qubo_search_step(None, 12, None, ctypes.byref(q.Progress(**good))) == q.QUBO_EINVAL
    assert lib.qubo_search_step(P, 12, None, None) == q.QUBO_EINVAL
    done = q.Progress(**good, done=1)
    before = bytes(done)
    assert lib.qubo_search_step(P, 12, None, ctypes.byref(done)) == q.QUBO_OK
    assert bytes(done) == before
    # binary64 runs: n from 5 to 58, no split; each kind's step refuses the other's record
    for n_, pb, cb in [(4, -1, -1), (59, -1, -1), (12, 8, 4), (12, 8, 9), (12, 13, -1)]:
        assert lib.qubo_progress_init_f64(P, n_, pb, cb, None, ctypes.byref(p)) == q.QUBO_EINVAL, (n_, pb, cb)
    assert lib.qubo_progress_init_f64(None, 12, -1, -1, None, ctypes.byref(p)) == q.QUBO_EINVAL
    assert lib.qubo_progress_init_f64(P, 12, -1, -1, None, None) == q.QUBO_EINVAL
    f_good = dict(good, kind=1)
    assert lib.qubo_search_step(P, 12, None, ctypes.byref(q.Progress(**f_good))) == q.QUBO_EINVAL
    assert lib.qubo_search_step_f64(P, 12, None, ctypes.byref(q.Progress(**good))) == q.QUBO_EINVAL
    for change in bad + [dict(split_bits=1)]:
        rec = q.Progress(**{**f_good, **change})
        before = bytes(rec)
        assert lib.qubo_search_step_f64(P, 12, None, ctypes.byref(rec)) == q.QUBO_EINVAL, change
        assert bytes(rec) == before
    done = q.Progress(**f_good, done=1)
    before = bytes(done)
    assert lib.qubo_search_step_f64(P, 12, None, ctypes.byref(done)) == q.QUBO_OK
    assert bytes(done) == before


def test_spectrum_progress_record_and_rejections():
    """The spectrum run's record: the 96-byte header, k, found and 64 states;
    malformed arguments and records are refused before any device call."""
    lib = q.load()
    assert ctypes.sizeof(q.ProgressLowest) == 1128
    assert (q.ProgressLowest.head.offset, q.ProgressLowest.k.offset, q.ProgressLowest.found.offset,
            q.ProgressLowest.states.offset) == (0, 96, 100, 104)
    P = ctypes.c_void_p(16)
    pl = q.ProgressLowest()
    for k in (0, 65):
        assert lib.qubo_progress_init_lowest(P, 12, k, -1, -1, 0, None, ctypes.byref(pl)) == q.QUBO_EINVAL
    assert lib.qubo_progress_init_lowest(P, 12, 4, -1, -1, 0, None, None) == q.QUBO_EINVAL
    assert lib.qubo_progress_init_lowest(None, 12, 4, -1, -1, 0, None, ctypes.byref(pl)) == q.QUBO_EINVAL
    assert lib.qubo_progress_init_lowest(P, 12, 4, 8, 4, 0, None, ctypes.byref(pl)) == q.QUBO_EINVAL
    assert bytes(pl) == bytes(1128)
    head = dict(n=12, split_bits=0, prefix_bits=8, chunk_bits=6, steps_total=4, kind=2)
    for h, k, found in [(dict(head, kind=0), 4, 0), (head, 0, 0), (head, 65, 0), (head, 4, 5), (head, 4, -1),
                        (dict(head, chunk_bits=9), 4, 0), (dict(head, n=13), 4, 0)]:
        rec = q.ProgressLowest(head=q.Progress(**h), k=k, found=found)
        before = bytes(rec)
        assert lib.qubo_search_step_lowest(P, 12, None, ctypes.byref(rec)) == q.QUBO_EINVAL, (h, k, found)
        assert bytes(rec) == before
    # a spectrum record is not a minimum record, and a finished run's step does nothing
    assert lib.qubo_search_step(P, 12, None, ctypes.byref(q.Progress(**head))) == q.QUBO_EINVAL
    done = q.ProgressLowest(head=q.Progress(**dict(head, done=1)), k=4)
    before = bytes(done)
    assert lib.qubo_search_step_lowest(P, 12, None, ctypes.byref(done)) == q.QUBO_OK
    assert bytes(done) == before


def test_timing_struct_before_any_search():
    t = q.last_timing()
    assert set(t) >= {"build_ms", "search_ms", "reduce_ms", "total_ms", "states", "slow_bodies"}
