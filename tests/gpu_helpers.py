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
