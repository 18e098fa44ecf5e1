"""A search run in slices (qubo_progress_init / qubo_search_step and their
binary64 forms): resumed from its 96-byte state it gives exactly the one-call
search's result, with and without the outer split (the straightforward split of
sec. III.C.1), and whole sub-problems above the best energy are skipped."""
from __future__ import annotations

import ctypes
import json
import os

import numpy as np
import pytest

import oracle
import qubo_instances as qi
from gpu_helpers import announce, dev_q

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


def run_all(q, Qd, p):
    states = 0
    while not p.done:
        q.search_step(Qd, p)
        states += q.last_timing()["states"]
    return states


def test_resume_from_bytes_n32(q):
    """C2 (n=32) in 8 slices, stopped after 3 and continued from a copy of the
    record's bytes: the stored oracle result, every state searched once."""
    with open(os.path.join(GOLDEN, "C2.json")) as f:
        g = json.load(f)
    cfg = qi.make_config("C2")
    Qd = dev_q(cfg["Q"])
    A = q.make_plan(32)["prefix_bits"]
    announce("resumable C2 init")
    p = q.progress_init(Qd, chunk_bits=A - 3)
    assert (p.n, p.split_bits, p.prefix_bits, p.steps_total, p.done) == (32, 0, A, 8, 0)
    states = 0
    for i in range(3):
        announce("resumable C2 step", i)
        assert not q.search_step(Qd, p)
        states += q.last_timing()["states"]
    saved = bytes(p)
    p2 = q.Progress.from_buffer_copy(saved)
    assert (p2.steps_done, p2.next, p2.sub) == (3, 3 << (A - 3), 0)
    announce("resumable C2 rest")
    states += run_all(q, Qd, p2)
    assert states == 1 << 32
    assert p2.steps_done == p2.steps_total == 8
    assert p2.result().triple() == (g["min_energy"], g["argmin"], g["count"])
    # a finished run's step changes nothing
    before = bytes(p2)
    assert q.search_step(Qd, p2)
    assert bytes(p2) == before


@pytest.mark.parametrize("n,k,seed", [(26, 2, 9101), (24, 3, 9102)])
def test_outer_split_in_slices(q, n, k, seed):
    Q = qi.general_uniform(n, seed, -100, 100)
    want = oracle.search_gray(Q).triple()
    Qd = dev_q(Q)
    announce("resumable split", n, k)
    A = 12  # 8 slices of 2^9 Gray steps per sub-problem
    p = q.progress_init(Qd, prefix_bits=A, chunk_bits=9, split_bits=k)
    assert (p.split_bits, p.prefix_bits, p.steps_total) == (k, A, (1 << k) << (A - 9))
    run_all(q, Qd, p)
    assert p.steps_done == p.steps_total
    assert p.result().triple() == want
    assert q.search(Qd, split_bits=k).triple() == want


def test_sub_problems_above_the_best_are_skipped(q):
    """Variable 0 costs +100000 when set: once the x_0 = 0 half is searched, the
    x_0 = 1 sub-problem lies wholly above the best energy and is skipped."""
    n = 22
    Q = np.array(qi.symmetric_uniform(n, 9103, -100, 100), dtype=np.int64)
    Q[0, 0] = 100000
    want = oracle.search_gray(Q.tolist()).triple()
    Qd = dev_q(Q)
    announce("resumable skip")
    p = q.progress_init(Qd, chunk_bits=q.make_plan(n - 1)["prefix_bits"], split_bits=1)
    assert p.steps_total == 2
    assert not q.search_step(Qd, p)
    assert q.last_timing()["states"] == 1 << (n - 1)
    assert q.search_step(Qd, p)
    assert q.last_timing()["states"] == 0  # skipped: nothing launched
    assert p.result().triple() == want


def test_other_matrix_refused(q):
    Q1 = qi.general_uniform(20, 9104, -50, 50)
    Q2 = [row[:] for row in Q1]
    Q2[3][7] += 1
    Qd1, Qd2 = dev_q(Q1), dev_q(Q2)
    announce("resumable fingerprint")
    p = q.progress_init(Qd1, prefix_bits=10, chunk_bits=6)
    before = bytes(p)
    with pytest.raises(q.QuboError) as e:
        q.search_step(Qd2, p)
    assert e.value.code == q.QUBO_EINVAL
    assert bytes(p) == before
    lib = q.load()
    assert lib.qubo_search_step(ctypes.c_void_p(Qd1.data_ptr()), 19, None, ctypes.byref(p)) == q.QUBO_EINVAL


def test_search_resumable_file(q, tmp_path):
    """The file-backed loop: interrupted after two steps, continued by a second
    call, and a finished file answers at once."""
    n = 28
    Q = qi.general_uniform(n, 9105, -100, 100)
    want = oracle.search_gray(Q).triple()
    Qd = dev_q(Q)
    path = str(tmp_path / "run.qubo")
    announce("resumable file")
    assert q.search_resumable(Qd, path, prefix_bits=16, chunk_bits=10, max_steps=2) is None
    assert os.path.getsize(path) == 96
    p = q.Progress.from_buffer_copy(open(path, "rb").read())
    assert p.steps_done == 2 and not p.done
    r = q.search_resumable(Qd, path)
    assert r.triple() == want
    assert q.search_resumable(Qd, path, max_steps=0).triple() == want


def test_first_step_of_n60(q):
    """n = 60 splits into 4 sub-problems of 58 variables (A = 32, B = 26). Its
    first step searches the first 2^22 Gray steps of x_0 = x_1 = 0, which is the
    58-variable problem of Q[2:, 2:] (nothing fixed is set): the same slice of
    that matrix gives the same result."""
    import torch
    n = 60
    Q = qi.symmetric_uniform(n, 9106, -100, 100)
    Qd = dev_q(Q)
    announce("resumable n=60 init")
    p = q.progress_init(Qd)
    assert (p.split_bits, p.prefix_bits, p.chunk_bits) == (2, 32, 22)
    assert p.steps_total == 4 << 10
    announce("resumable n=60 step")
    assert not q.search_step(Qd, p)
    assert (p.sub, p.next, p.steps_done) == (0, 1 << 22, 1)
    sub = Qd[2:, 2:].contiguous()
    announce("n=58 slice of Q[2:, 2:]")
    r = q.search_range(sub, 32, 0, 1 << 22)
    assert p.result().triple() == r.triple()
    del sub
    torch.cuda.synchronize()


def test_resume_f64_from_bytes_n32(q):
    """The real-valued n = 32 workload (C2f) in 8 slices, stopped
    after 3 and continued from the record's bytes: the stored oracle result."""
    import torch
    with open(os.path.join(GOLDEN, "C2f.json")) as f:
        g = json.load(f)
    cfg = qi.make_config("C2f")
    assert qi.sha256_of(cfg["Q"]) == g["sha256_Q"]
    Qd = torch.as_tensor(np.asarray(cfg["Q"], dtype=np.float64)).to("cuda:0").contiguous()
    announce("resumable C2f init")
    p = q.progress_init(Qd, chunk_bits=q.make_plan(32)["prefix_bits"] - 3)
    assert (p.kind, p.split_bits, p.steps_total) == (1, 0, 8)
    for i in range(3):
        announce("resumable C2f step", i)
        q.search_step(Qd, p)
    p2 = q.Progress.from_buffer_copy(bytes(p))
    announce("resumable C2f rest")
    while not q.search_step(Qd, p2):
        pass
    r = p2.result()
    assert (float.hex(r.min_energy), r.argmin, r.count) == (g["min_energy_hex"], g["argmin"], g["count"])
    with pytest.raises(q.QuboError) as e:  # an int32 step refuses a binary64 record
        q.search_step(dev_q(np.zeros((32, 32))), p2)
    assert e.value.code == q.QUBO_EINVAL


def test_search_resumable_file_f64(q, tmp_path):
    import torch
    n = 20
    rng = np.random.default_rng(9301)
    Q = rng.uniform(-10.0, 10.0, size=(n, n))
    want = oracle.search_direct_f64(Q).triple()
    Qd = torch.as_tensor(Q).to("cuda:0").contiguous()
    path = str(tmp_path / "run_f64.qubo")
    announce("resumable file f64")
    assert q.search_resumable(Qd, path, prefix_bits=10, chunk_bits=6, max_steps=3) is None
    assert q.search_resumable(Qd, path).triple() == want


def test_spectrum_run_resumed_n32(q):
    """The 64 lowest states of C2 (n=32) in 8 slices, stopped after 3 and
    continued from the record's bytes: the stored oracle list."""
    with open(os.path.join(GOLDEN, "C2low.json")) as f:
        g = json.load(f)
    cfg = qi.make_config("C2")
    assert qi.sha256_of(cfg["Q"]) == g["sha256_Q"]
    Qd = dev_q(cfg["Q"])
    A = q.make_plan(32)["prefix_bits"]
    announce("spectrum run C2 init")
    p = q.progress_init(Qd, chunk_bits=A - 3, k=64)
    assert (p.head.kind, p.k, p.found, p.head.steps_total) == (2, 64, 0, 8)
    for i in range(3):
        announce("spectrum run C2 step", i)
        assert not q.search_step(Qd, p)
    p2 = q.ProgressLowest.from_buffer_copy(bytes(p))
    announce("spectrum run C2 rest")
    while not q.search_step(Qd, p2):
        pass
    assert p2.result() == [(int(e), int(i)) for e, i in g["states"]]
    assert p2.result() == q.lowest(Qd, 64)


@pytest.mark.parametrize("n,k,seed", [(24, 2, 9401), (22, 3, 9402)])
def test_spectrum_run_split(q, n, k, seed):
    Q = qi.general_uniform(n, seed, -3, 3)  # heavy ties: the list's order decides
    want = [tuple(map(int, s)) for s in oracle.lowest(Q, 40)]
    Qd = dev_q(Q)
    announce("spectrum run split", n, k)
    p = q.progress_init(Qd, prefix_bits=12, chunk_bits=9, split_bits=k, k=40)
    while not q.search_step(Qd, p):
        pass
    assert p.head.steps_done == p.head.steps_total == (1 << k) << 3
    assert p.result() == want


def test_spectrum_run_skips_sub_problems(q, tmp_path):
    """With +100000 on variable 0, once the x_0 = 0 half has filled the list,
    the x_0 = 1 sub-problem lies above its 8th energy and is skipped; the file
    loop gives the same list."""
    n = 22
    Q = np.array(qi.symmetric_uniform(n, 9403, -100, 100), dtype=np.int64)
    Q[0, 0] = 100000
    want = [tuple(map(int, s)) for s in oracle.lowest(Q.tolist(), 8)]
    Qd = dev_q(Q)
    announce("spectrum run skip")
    p = q.progress_init(Qd, chunk_bits=q.make_plan(n - 1)["prefix_bits"], split_bits=1, k=8)
    assert not q.search_step(Qd, p)
    assert q.search_step(Qd, p)
    assert q.last_timing()["states"] == 0  # skipped: nothing launched
    assert p.result() == want
    path = str(tmp_path / "spectrum.qubo")
    assert q.search_resumable(Qd, path, split_bits=1, k=8, max_steps=1) is None
    assert os.path.getsize(path) == 1128
    assert q.search_resumable(Qd, path, split_bits=1, k=8) == want
