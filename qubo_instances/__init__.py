"""Seeded synthetic QUBO instances shared by the oracle's tests, the GPU tests and bench.py.

This module only draws random numbers and assembles matrices.  It evaluates no
energy, folds nothing and searches nothing: none of the solver's arithmetic
lives here, so the CPU oracle and the HIP path can both take their inputs from
it without sharing any of the method.

Conventions (Maltsev et al., "Terastate-per-second QUBO Brute-Force on a Single
GPU", sec. I: E(x) = sum_ij Q_ij x_i x_j over x in {0,1}^n):
  * a matrix is a list of n rows of n Python ints (row-major), or a numpy int32
    array via ``as_array``;
  * a state is the integer idx = sum_i x_i 2^(n-1-i) (variable 0 is the most
    significant bit, the lexicographic row order of the state matrix U_N in
    sec. II.B, Fig. 2).

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), written from its published
description: add the golden-gamma increment, then two xor-shift-multiply
rounds and a final xor-shift.
"""
from __future__ import annotations

import hashlib
import math
import struct

MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB


class SplitMix64:
    """SplitMix64 stream: state advances by the golden gamma; output is mixed."""

    def __init__(self, seed: int):
        self.state = seed & MASK64

    def next_u64(self) -> int:
        self.state = (self.state + _GAMMA) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * _MIX1) & MASK64
        z = ((z ^ (z >> 27)) * _MIX2) & MASK64
        return z ^ (z >> 31)

    def uniform_int(self, lo: int, hi: int) -> int:
        """Uniform integer in [lo, hi] by rejection (no modulo bias)."""
        span = hi - lo + 1
        if span <= 0:
            raise ValueError("empty range")
        limit = (1 << 64) - ((1 << 64) % span)
        while True:
            r = self.next_u64()
            if r < limit:
                return lo + (r % span)

    def uniform01(self) -> float:
        """53-bit uniform double in [0, 1)."""
        return (self.next_u64() >> 11) * (1.0 / (1 << 53))

    def normal(self) -> float:
        """Standard normal by Box-Muller (one output per pair of uniforms)."""
        u1 = 1.0 - self.uniform01()          # (0, 1]: log is finite
        u2 = self.uniform01()
        return math.sqrt(-2.0 * math.log(u1)) * math.cos(2.0 * math.pi * u2)


def zeros(n: int) -> list[list[int]]:
    return [[0] * n for _ in range(n)]


def symmetric_uniform(n: int, seed: int, lo: int, hi: int,
                      diag_lo: int | None = None, diag_hi: int | None = None) -> list[list[int]]:
    """Symmetric Q: the upper triangle (i <= j) is drawn row-major and mirrored.

    Off-diagonal entries are uniform in [lo, hi]; diagonal entries are uniform in
    [diag_lo, diag_hi] (default: the same range).
    """
    if diag_lo is None:
        diag_lo, diag_hi = lo, hi
    rng = SplitMix64(seed)
    q = zeros(n)
    for i in range(n):
        for j in range(i, n):
            v = rng.uniform_int(diag_lo, diag_hi) if i == j else rng.uniform_int(lo, hi)
            q[i][j] = v
            q[j][i] = v
    return q


def general_uniform(n: int, seed: int, lo: int, hi: int) -> list[list[int]]:
    """Non-symmetric Q with every entry drawn independently, row-major."""
    rng = SplitMix64(seed)
    return [[rng.uniform_int(lo, hi) for _ in range(n)] for _ in range(n)]


def _real(rng: SplitMix64, lo: float, hi: float) -> float:
    return lo + (hi - lo) * rng.uniform01()


def symmetric_uniform_f64(n: int, seed: int, lo: float, hi: float) -> list[list[float]]:
    """Real symmetric Q (binary64): upper triangle drawn row-major, uniform in
    [lo, hi), and mirrored."""
    rng = SplitMix64(seed)
    q = [[0.0] * n for _ in range(n)]
    for i in range(n):
        for j in range(i, n):
            v = _real(rng, lo, hi)
            q[i][j] = v
            q[j][i] = v
    return q


def general_uniform_f64(n: int, seed: int, lo: float, hi: float) -> list[list[float]]:
    """Real non-symmetric Q (binary64), every entry uniform in [lo, hi), row-major."""
    rng = SplitMix64(seed)
    return [[_real(rng, lo, hi) for _ in range(n)] for _ in range(n)]


def ising_to_qubo(J: list[list[int]], h: list[int]) -> tuple[list[list[int]], int]:
    """Map H(s) = sum_{i<j} J_ij s_i s_j + sum_i h_i s_i (s = 2x - 1) to a QUBO.

    Returns (Q, C) with a symmetric Q such that H(s) = E_Q(x) + C, where
    Q_ij = Q_ji = 2 J_ij (i != j), Q_ii = 2 h_i - 2 sum_{j != i} J_ij and
    C = sum_{i<j} J_ij - sum_i h_i.  Only J's upper triangle (i < j) is read.
    This is substitution s_i s_j = 4 x_i x_j - 2 x_i - 2 x_j + 1, s_i = 2 x_i - 1,
    with the linear terms moved onto the diagonal (x_i^2 = x_i).
    """
    n = len(h)
    q = zeros(n)
    c = 0
    for i in range(n):
        for j in range(i + 1, n):
            jij = J[i][j]
            q[i][j] = 2 * jij
            q[j][i] = 2 * jij
            q[i][i] -= 2 * jij
            q[j][j] -= 2 * jij
            c += jij
    for i in range(n):
        q[i][i] += 2 * h[i]
        c -= h[i]
    return q, c


def sk_pm1(n: int, seed: int) -> tuple[list[list[int]], list[int]]:
    """Sherrington-Kirkpatrick +-1 couplings: J_ij in {-1, +1} for i < j, h = 0."""
    rng = SplitMix64(seed)
    J = zeros(n)
    for i in range(n):
        for j in range(i + 1, n):
            J[i][j] = 2 * rng.uniform_int(0, 1) - 1
    return J, [0] * n


def mattis(n: int, seed: int) -> tuple[list[list[int]], list[int], list[int]]:
    """Mattis instance J_ij = -xi_i xi_j (i < j), h = 0, xi in {-1,+1}^n drawn from the seed.

    Its ground states are s = xi and s = -xi with H = -n(n-1)/2.
    Returns (J, h, xi).
    """
    rng = SplitMix64(seed)
    xi = [2 * rng.uniform_int(0, 1) - 1 for _ in range(n)]
    J = zeros(n)
    for i in range(n):
        for j in range(i + 1, n):
            J[i][j] = -xi[i] * xi[j]
    return J, [0] * n, xi


def gauge_transform(p: list[list[int]], a: list[int]) -> list[list[int]]:
    """Matrix of x -> E_P(x xor a) - E_P(a) (a change of variables, no search).

    With y = x xor a, y_i = a_i + b_i x_i where b_i = 1 - 2 a_i; expanding
    sum_ij P_ij y_i y_j and using x_i^2 = x_i gives
        Q_ij = b_i b_j P_ij (i != j),  Q_ii = b_i P_ii + b_i sum_{j != i} a_j (P_ij + P_ji),
    and the constant E_P(a), which is dropped.
    """
    n = len(a)
    b = [1 - 2 * ai for ai in a]
    q = zeros(n)
    for i in range(n):
        for j in range(n):
            if i != j:
                q[i][j] = b[i] * b[j] * p[i][j]
        q[i][i] = b[i] * p[i][i] + b[i] * sum(a[j] * (p[i][j] + p[j][i]) for j in range(n) if j != i)
    return q


def planted(n: int, seed: int, off_hi: int = 100, diag_lo: int = 1, diag_hi: int = 200):
    """Instance with a seed-chosen unique minimiser x*.

    Draws x* (n bits), then a symmetric P with off-diagonal entries uniform in
    [0, off_hi] and diagonal entries uniform in [diag_lo, diag_hi] (diag_lo >= 1),
    so that E_P(y) > 0 for every y != 0 and y = 0 is P's unique minimiser.  Q is
    gauge_transform(P, x*): E_Q(x) = E_P(x xor x*) - E_P(x*), whose unique
    minimiser is x = x* with energy -E_P(x*).  Returns (Q, P, xstar_bits); the
    expected minimum is left for the caller to evaluate.
    """
    if diag_lo < 1:
        raise ValueError("diag_lo must be >= 1 so that x* is the unique minimiser")
    rng = SplitMix64(seed)
    a = [rng.uniform_int(0, 1) for _ in range(n)]
    p = symmetric_uniform(n, rng.next_u64(), 0, off_hi, diag_lo, diag_hi)
    return gauge_transform(p, a), p, a


def round_half_away(v: float) -> int:
    return int(math.floor(v + 0.5)) if v >= 0 else -int(math.floor(-v + 0.5))


def low_rank_noise(n: int, seed: int, rank: int = 4, scale: float = 10.0, noise: int = 20) -> list[list[int]]:
    """Q = round(scale * U U^T) + N with U n x rank standard normal (row-major draws)
    and N symmetric uniform in [-noise, noise] drawn for i <= j after U.

    The product is summed in double over k = 0..rank-1 in order and rounded half
    away from zero; the diagonal is included.
    """
    rng = SplitMix64(seed)
    u = [[rng.normal() for _ in range(rank)] for _ in range(n)]
    q = zeros(n)
    for i in range(n):
        for j in range(i, n):
            acc = 0.0
            for k in range(rank):
                acc += u[i][k] * u[j][k]
            v = round_half_away(scale * acc) + rng.uniform_int(-noise, noise)
            q[i][j] = v
            q[j][i] = v
    return q


# Named workloads.  Each returns a dict with the matrix and whatever the caller
# needs to state expectations that do not come from running a solver.
CONFIGS = {
    "C1": dict(n=24, seed=1001, desc="dense QUBO n=24, symmetric, all entries uniform in [-100,100]"),
    "C2": dict(n=32, seed=1002, desc="dense QUBO n=32, symmetric, off-diagonal uniform in [-100,100], diagonal in [-200,200]"),
    "C2p": dict(n=32, seed=1102, desc="planted QUBO n=32: unique seed-chosen minimiser"),
    "C3": dict(n=40, seed=1003, desc="+-1 Sherrington-Kirkpatrick n=40, h=0, as an int32 QUBO via x=(1+s)/2"),
    "C4": dict(n=48, seed=1004, desc="dense QUBO n=48, symmetric, all entries uniform in [-100,100]"),
    "C5": dict(n=50, seed=1005, desc="dense QUBO n=50, round(10 U U^T) + uniform[-20,20] noise, U 50x4 standard normal"),
    # the largest single-launch size (A = 32, B = 26 at the default split)
    "C58": dict(n=58, seed=1058, desc="dense QUBO n=58, symmetric, all entries uniform in [-100,100]"),
    # real-valued (binary64) counterparts of C1, C2 and C4
    "C1f": dict(n=24, seed=1011, desc="dense real QUBO n=24, symmetric, binary64 entries uniform in [-100,100)"),
    "C2f": dict(n=32, seed=1012, desc="dense real QUBO n=32, symmetric, binary64 entries uniform in [-100,100)"),
    "C4f": dict(n=48, seed=1014, desc="dense real QUBO n=48, symmetric, binary64 entries uniform in [-100,100)"),
}


def make_config(name: str) -> dict:
    """Build one named workload.  Keys: name, n, Q, desc, plus family extras
    (planted: P, xstar; SK: J, h, C)."""
    spec = CONFIGS[name]
    n, seed = spec["n"], spec["seed"]
    out = dict(name=name, n=n, desc=spec["desc"], seed=seed)
    if name in ("C1", "C4", "C58"):
        out["Q"] = symmetric_uniform(n, seed, -100, 100)
    elif name == "C2":
        out["Q"] = symmetric_uniform(n, seed, -100, 100, -200, 200)
    elif name == "C2p":
        q, p, a = planted(n, seed)
        out.update(Q=q, P=p, xstar=a)
    elif name == "C3":
        J, h = sk_pm1(n, seed)
        q, c = ising_to_qubo(J, h)
        out.update(Q=q, J=J, h=h, C=c)
    elif name == "C5":
        out["Q"] = low_rank_noise(n, seed)
    elif name in ("C1f", "C2f", "C4f"):
        out["Q"] = symmetric_uniform_f64(n, seed, -100.0, 100.0)
    else:
        raise KeyError(name)
    return out


def bits_to_index(bits: list[int]) -> int:
    """idx = sum_i x_i 2^(n-1-i): variable 0 is the most significant bit."""
    idx = 0
    for b in bits:
        idx = (idx << 1) | (b & 1)
    return idx


def index_to_bits(idx: int, n: int) -> list[int]:
    return [(idx >> (n - 1 - i)) & 1 for i in range(n)]


def as_array(q):
    """numpy int32 copy of a list-of-rows matrix (import deferred so the module
    itself needs only the standard library)."""
    import numpy as np
    return np.asarray(q, dtype=np.int32)


def sha256_of(q) -> str:
    """SHA-256 of the little-endian row-major bytes of Q: int32 entries, or
    binary64 when the entries are floats."""
    n = len(q)
    fmt = "<%dd" % n if isinstance(q[0][0], float) else "<%di" % n
    buf = b"".join(struct.pack(fmt, *row) for row in q)
    return hashlib.sha256(buf).hexdigest()
