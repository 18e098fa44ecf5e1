"""Shared helpers for the GPU tests: device tensors and case announcements."""
from __future__ import annotations

import sys

import numpy as np


def announce(*what):
    """Print the case about to run on the GPU, flushed, so a fault names it."""
    print("[gpu case]", *what, file=sys.stderr, flush=True)


def dev_q(Q):
    import torch
    return torch.as_tensor(np.asarray(Q, dtype=np.int32)).to("cuda:0").contiguous()


def gray(i: int) -> int:
    return i ^ (i >> 1)


def inv_gray(g: int) -> int:
    """j with gray(j) == g (prefix xor over the bits of g)."""
    j = 0
    while g:
        j ^= g
        g >>= 1
    return j


def check_coverage(q, n, prefix_bits=None, cache_bits=None, lo=None, hi=None, strict=False,
                   cols_per_lane=None):
    """The last search walked every 32-step body of its range exactly once per
    column group: bodies * 32 * 64R == (hi - lo) * (2^B padded to 64R columns),
    R the columns per lane that the search reports (and, when given, asked for)."""
    plan = q.make_plan(n, prefix_bits, cache_bits)
    A, B = plan["prefix_bits"], plan["suffix_bits"]
    t = q.last_timing()
    R = t["cols_per_lane"]
    assert cols_per_lane in (None, R), (cols_per_lane, t)
    group = 64 * R
    cols_padded = -(-(1 << B) // group) * group
    lo = 0 if lo is None else lo
    hi = (1 << A) if hi is None else hi
    assert t["bodies"] * 32 * group == (hi - lo) * cols_padded, (t, plan, R)
    if strict:
        assert t["checked_bodies"] == t["bodies"], t
    assert t["slow_bodies"] <= t["checked_bodies"] <= t["bodies"], t
