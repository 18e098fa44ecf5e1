"""qubo_search_noalloc -- the int32 search that allocates no device memory --
against qubo_search, the entry point it is a variant of.

The no-allocation search keeps its workspace in one static 128 MiB device buffer
per GPU, which keeps the last call's contents; each call must build everything
it reads itself.  So the checks run calls back to back with different sizes
(the second smaller than the first), on the default and on another stream,
and compare each with qubo_search bit for bit (minimum, lowest minimiser,
count), and the stored whole-space oracle results where there are any.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import qubo_instances as qi
from gpu_helpers import announce, check_coverage, dev_q

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


def stored(name):
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        g = json.load(f)
    return (g["min_energy"], g["argmin"], g["count"])


def test_back_to_back_sizes(q):
    """n = 40, then n = 32, then n = 24, then n = 3 (padded to 5 variables):
    each call after a larger one, whose tables, partials and counters are still
    in the buffer."""
    names = ["C3", "C2", "C1"]
    mats = [qi.make_config(name)["Q"] for name in names] + [qi.general_uniform(3, 9901, -5, 5)]
    devs = [dev_q(Q) for Q in mats]
    want = []
    for i, Qd in enumerate(devs):
        announce("no-alloc reference search", i)
        want.append(q.search(Qd).triple())
    for name, w in zip(names, want):
        assert w == stored(name), name
    for rnd in range(2):
        for i, Qd in enumerate(devs):
            announce("no-alloc search", rnd, i)
            assert q.search_noalloc(Qd).triple() == want[i], (rnd, i)
            n = int(Qd.shape[0])
            if n >= 5:
                check_coverage(q, n)


def test_explicit_split_and_stream(q):
    """A split other than the planner's (n = 42 at 24 prefix bits, 90 MiB of
    the buffer), then a smaller search on a stream of its own, then the first
    again: each equals qubo_search with the same arguments."""
    import torch
    Qa = dev_q(qi.general_uniform(42, 9902, -100, 100))
    Qb = dev_q(qi.general_uniform(30, 9903, -3, 3))  # heavy ties: counts well above 1
    announce("no-alloc reference n=42 A=24")
    wa = q.search(Qa, prefix_bits=24, cache_bits=12).triple()
    announce("no-alloc reference n=30")
    wb = q.search(Qb).triple()
    announce("no-alloc n=42 A=24")
    assert q.search_noalloc(Qa, prefix_bits=24, cache_bits=12).triple() == wa
    check_coverage(q, 42, 24, 12)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        announce("no-alloc n=30 other stream")
        assert q.search_noalloc(Qb, stream=s).triple() == wb
    s.synchronize()
    announce("no-alloc n=42 A=24 again")
    assert q.search_noalloc(Qa, prefix_bits=24, cache_bits=12).triple() == wa


def test_too_large_is_rejected(q):
    """A plan whose workspace exceeds the buffer is refused before any device
    work, and the next call still gives the right answer."""
    Q48 = dev_q(qi.make_config("C4")["Q"])
    announce("no-alloc n=48 rejected")
    with pytest.raises(q.QuboError) as e:
        q.search_noalloc(Q48)
    assert e.value.code == q.QUBO_ESCRATCH
    assert "128 MiB" in q.strerror(q.QUBO_ESCRATCH)
    Q2 = dev_q(qi.make_config("C2")["Q"])
    announce("no-alloc n=32 after the rejection")
    assert q.search_noalloc(Q2).triple() == stored("C2")
    with pytest.raises(q.QuboError) as e:
        q.search_noalloc(dev_q(np.array([[2 ** 30, 0], [0, 0]])))
    assert e.value.code == q.QUBO_ERANGE
