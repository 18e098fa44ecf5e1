"""CPU oracle for exhaustive QUBO search -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The solver never does, and this package
imports nothing from the solver: it shares no code, header, table or helper with
the HIP path.  Its inputs come from ``qubo_instances`` (random draws only).

The arithmetic lives in ``oracle.c`` (plain C, int64; binary64 for a
floating-point Q, summed in a fixed row-major order): the definition
E(x) = sum_ij Q_ij x_i x_j of Maltsev et al., "Terastate-per-second QUBO
Brute-Force on a Single GPU", sec. I, evaluated directly (tier A) and by an
incremental Gray-code walk (tier B, sec. I.D).  This module only marshals
arguments through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")

# Baseline x86-64 with AVX2: the library is built here and also loaded on other
# hosts, so it must not assume the build host's newest vector extensions.
CFLAGS = ["-O3", "-march=x86-64-v3", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread"]


def build(out_path: str = LIB_PATH, defines: tuple[str, ...] = (), verbose: bool = False) -> str:
    """Compile oracle.c with gcc into ``out_path`` (always recompiles)."""
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *["-D" + d for d in defines], SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


class _Result(ctypes.Structure):
    _fields_ = [("min_energy", ctypes.c_int64), ("argmin", ctypes.c_uint64),
                ("count", ctypes.c_uint64), ("max_abs_energy", ctypes.c_int64)]


@dataclass(frozen=True)
class Result:
    min_energy: int
    argmin: int
    count: int
    max_abs_energy: int

    def triple(self) -> tuple[int, int, int]:
        return (self.min_energy, self.argmin, self.count)


class _ResultF64(ctypes.Structure):
    _fields_ = [("min_energy", ctypes.c_double), ("argmin", ctypes.c_uint64),
                ("count", ctypes.c_uint64), ("max_abs_energy", ctypes.c_double)]


@dataclass(frozen=True)
class ResultF64:
    min_energy: float
    argmin: int
    count: int
    max_abs_energy: float

    def triple(self) -> tuple[float, int, int]:
        return (self.min_energy, self.argmin, self.count)


def _farray(Q) -> np.ndarray:
    q = np.ascontiguousarray(np.asarray(Q, dtype=np.float64))
    if q.ndim != 2 or q.shape[0] != q.shape[1]:
        raise ValueError("Q must be square")
    return q


def _fptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _qarray(Q) -> np.ndarray:
    q = np.asarray(Q, dtype=np.int64)
    if q.ndim != 2 or q.shape[0] != q.shape[1]:
        raise ValueError("Q must be square")
    if q.size and (q.min() < -(2 ** 31) or q.max() > 2 ** 31 - 1):
        raise ValueError("Q entries must fit int32")
    return np.ascontiguousarray(q.astype(np.int32))


def _ptr(q: np.ndarray):
    return q.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


class Oracle:
    """One loaded build of oracle.c (the default build, or a mutant for pin tests)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_energy.argtypes = [i32p, ctypes.c_int, ctypes.c_uint64]
        lib.oracle_energy.restype = ctypes.c_int64
        lib.oracle_energy_many.argtypes = [i32p, ctypes.c_int, ctypes.POINTER(ctypes.c_uint64),
                                           ctypes.c_uint64, ctypes.POINTER(ctypes.c_int64)]
        lib.oracle_energy_many.restype = None
        lib.oracle_search_direct.argtypes = [i32p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                             ctypes.c_int, ctypes.POINTER(_Result)]
        lib.oracle_search_direct.restype = ctypes.c_int
        lib.oracle_search_gray.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                           ctypes.c_int, ctypes.POINTER(_Result)]
        lib.oracle_search_gray.restype = ctypes.c_int
        lib.oracle_lowest.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_uint64, ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                      ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_int)]
        lib.oracle_lowest.restype = ctypes.c_int
        f64p = ctypes.POINTER(ctypes.c_double)
        lib.oracle_energy_f64.argtypes = [f64p, ctypes.c_int, ctypes.c_uint64]
        lib.oracle_energy_f64.restype = ctypes.c_double
        lib.oracle_energy_many_f64.argtypes = [f64p, ctypes.c_int, ctypes.POINTER(ctypes.c_uint64),
                                               ctypes.c_uint64, f64p]
        lib.oracle_energy_many_f64.restype = None
        lib.oracle_search_direct_f64.argtypes = [f64p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                                 ctypes.c_int, ctypes.POINTER(_ResultF64)]
        lib.oracle_search_direct_f64.restype = ctypes.c_int
        lib.oracle_lowest_f64.argtypes = [f64p, ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_int, f64p, ctypes.POINTER(ctypes.c_uint64),
                                          ctypes.POINTER(ctypes.c_int)]
        lib.oracle_lowest_f64.restype = ctypes.c_int
        lib.oracle_version.restype = ctypes.c_char_p
        self.lib = lib
        self.path = path

    def energy(self, Q, idx: int) -> int:
        """E(x) for the state with index idx (variable 0 = most significant bit)."""
        q = _qarray(Q)
        return int(self.lib.oracle_energy(_ptr(q), q.shape[0], int(idx)))

    def energies(self, Q, idx) -> np.ndarray:
        q = _qarray(Q)
        ids = np.ascontiguousarray(np.asarray(idx, dtype=np.uint64))
        out = np.empty(ids.shape, dtype=np.int64)
        self.lib.oracle_energy_many(_ptr(q), q.shape[0],
                                    ids.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), ids.size,
                                    out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        return out

    def search_direct(self, Q, lo: int = 0, hi: int | None = None, threads: int | None = None) -> Result:
        """Tier A: every index in [lo, hi) evaluated from the definition."""
        q = _qarray(Q)
        n = q.shape[0]
        if hi is None:
            hi = 1 << n
        r = _Result()
        rc = self.lib.oracle_search_direct(_ptr(q), n, lo, hi, threads or default_threads(), ctypes.byref(r))
        if rc != 0:
            raise ValueError("oracle_search_direct failed (%d)" % rc)
        return Result(r.min_energy, r.argmin, r.count, r.max_abs_energy)

    def search_gray(self, Q, k: int = 0, top: int = 0, threads: int | None = None) -> Result:
        """Tier B: Gray-code walk over the sub-cube whose first k variables spell `top`."""
        q = _qarray(Q)
        r = _Result()
        rc = self.lib.oracle_search_gray(_ptr(q), q.shape[0], k, top, threads or default_threads(),
                                         ctypes.byref(r))
        if rc != 0:
            raise ValueError("oracle_search_gray failed (%d)" % rc)
        return Result(r.min_energy, r.argmin, r.count, r.max_abs_energy)

    def lowest(self, Q, k: int, gray_walk: bool = True, threads: int | None = None, fixed: int = 0,
               top: int = 0) -> list[tuple[int, int]]:
        """The k lowest states as (E, index) pairs, ordered by E then index, of
        the sub-cube whose first `fixed` variables spell `top` (default: all)."""
        q = _qarray(Q)
        e = np.zeros(k, dtype=np.int64)
        ix = np.zeros(k, dtype=np.uint64)
        found = ctypes.c_int(0)
        rc = self.lib.oracle_lowest(_ptr(q), q.shape[0], k, 1 if gray_walk else 0, fixed, top,
                                    threads or default_threads(),
                                    e.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    ix.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), ctypes.byref(found))
        if rc != 0:
            raise ValueError("oracle_lowest failed (%d)" % rc)
        return [(int(e[i]), int(ix[i])) for i in range(found.value)]

    def energy_f64(self, Q, idx: int) -> float:
        """E(x) of a float64 Q, summed in the fixed row-major order."""
        q = _farray(Q)
        return float(self.lib.oracle_energy_f64(_fptr(q), q.shape[0], int(idx)))

    def energies_f64(self, Q, idx) -> np.ndarray:
        q = _farray(Q)
        ids = np.ascontiguousarray(np.asarray(idx, dtype=np.uint64))
        out = np.empty(ids.shape, dtype=np.float64)
        self.lib.oracle_energy_many_f64(_fptr(q), q.shape[0],
                                        ids.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), ids.size,
                                        _fptr(out))
        return out

    def search_direct_f64(self, Q, lo: int = 0, hi: int | None = None, threads: int | None = None) -> ResultF64:
        """Tier A for a float64 Q over the indices [lo, hi)."""
        q = _farray(Q)
        n = q.shape[0]
        if hi is None:
            hi = 1 << n
        r = _ResultF64()
        rc = self.lib.oracle_search_direct_f64(_fptr(q), n, lo, hi, threads or default_threads(), ctypes.byref(r))
        if rc != 0:
            raise ValueError("oracle_search_direct_f64 failed (%d)" % rc)
        return ResultF64(r.min_energy, r.argmin, r.count, r.max_abs_energy)

    def lowest_f64(self, Q, k: int, lo: int = 0, hi: int | None = None,
                   threads: int | None = None) -> list[tuple[float, int]]:
        """Tier A for a float64 Q: the k lowest states of the indices [lo, hi)
        as (E, index) pairs, ordered by E then index."""
        q = _farray(Q)
        n = q.shape[0]
        if hi is None:
            hi = 1 << n
        e = np.zeros(k, dtype=np.float64)
        ix = np.zeros(k, dtype=np.uint64)
        found = ctypes.c_int(0)
        rc = self.lib.oracle_lowest_f64(_fptr(q), n, k, lo, hi, threads or default_threads(), _fptr(e),
                                        ix.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), ctypes.byref(found))
        if rc != 0:
            raise ValueError("oracle_lowest_f64 failed (%d)" % rc)
        return [(float(e[i]), int(ix[i])) for i in range(found.value)]

    def version(self) -> str:
        return self.lib.oracle_version().decode()


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def energy(Q, idx: int) -> int:
    return default().energy(Q, idx)


def energies(Q, idx) -> np.ndarray:
    return default().energies(Q, idx)


def search_direct(Q, lo: int = 0, hi: int | None = None, threads: int | None = None) -> Result:
    return default().search_direct(Q, lo, hi, threads)


def search_gray(Q, k: int = 0, top: int = 0, threads: int | None = None) -> Result:
    return default().search_gray(Q, k, top, threads)


def lowest(Q, k: int, gray_walk: bool = True, threads: int | None = None, fixed: int = 0,
           top: int = 0) -> list[tuple[int, int]]:
    return default().lowest(Q, k, gray_walk, threads, fixed, top)


def energy_f64(Q, idx: int) -> float:
    return default().energy_f64(Q, idx)


def energies_f64(Q, idx) -> np.ndarray:
    return default().energies_f64(Q, idx)


def search_direct_f64(Q, lo: int = 0, hi: int | None = None, threads: int | None = None) -> ResultF64:
    return default().search_direct_f64(Q, lo, hi, threads)


def lowest_f64(Q, k: int, lo: int = 0, hi: int | None = None,
               threads: int | None = None) -> list[tuple[float, int]]:
    return default().lowest_f64(Q, k, lo, hi, threads)


def version() -> str:
    return default().version()
