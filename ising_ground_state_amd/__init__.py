"""Exhaustive dense-QUBO search on AMD Instinct MI355X (gfx950).

Thin ctypes binding of the C-ABI in ``include/qubo.h`` (``lib/libqubo.so``).
PyTorch supplies device memory and the current HIP stream; every step of the
search runs in the library's HIP kernels.  The binding fails loudly when the
library is missing: there is no CPU fallback.

    import torch, ising_ground_state_amd as q
    Q = torch.tensor(..., dtype=torch.int32, device="cuda")
    r = q.search(Q)            # r.min_energy, r.argmin, r.count
    low = q.lowest(Q, 10)      # the 10 lowest (energy, index) pairs

Method: Maltsev et al., "Terastate-per-second QUBO Brute-Force on a Single GPU:
A Matrix Prefix-Suffix Decomposition" (prefix-suffix split, sec. II; Gray-code
prefix walk, sec. III.B; parallel splits, sec. III.C).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libqubo.so")

QUBO_OK = 0
QUBO_EINVAL = -1
QUBO_ERANGE = -2
QUBO_EPLAN = -3
QUBO_EDEVICE = -4
QUBO_ENOMEM = -5
QUBO_ESCRATCH = -6
MAX_N = 63


class QuboError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        msg = "%s (status %d)" % (strerror(code) if _lib is not None else "qubo error", code)
        super().__init__(what + ": " + msg if what else msg)


class _Result(ctypes.Structure):
    _fields_ = [("min_energy", ctypes.c_int32), ("reserved", ctypes.c_uint32),
                ("argmin", ctypes.c_uint64), ("count", ctypes.c_uint64)]


class _ResultF64(ctypes.Structure):
    _fields_ = [("min_energy", ctypes.c_double), ("argmin", ctypes.c_uint64), ("count", ctypes.c_uint64)]


class _State(ctypes.Structure):
    _fields_ = [("energy", ctypes.c_int32), ("reserved", ctypes.c_uint32), ("index", ctypes.c_uint64)]


class _StateF64(ctypes.Structure):
    _fields_ = [("energy", ctypes.c_double), ("index", ctypes.c_uint64)]


class _Plan(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("n", "n_search", "prefix_bits", "suffix_bits", "cache_bits", "reg_bits",
                 "cols_per_lane", "wave_size", "waves_per_block", "seg_bits", "blocks", "lds_bytes",
                 "split_bits", "reserved")] + \
               [(name, ctypes.c_uint64) for name in ("col_groups", "work_units", "workspace_bytes")]


class _Best(ctypes.Union):
    _fields_ = [("best", _Result), ("best_f64", _ResultF64)]


class Progress(ctypes.Structure):
    """The state of a search run in slices (``qubo_progress``, 96 bytes): keep it
    between steps, e.g. as ``bytes(progress)`` in a file.  kind 0: int32 Q,
    kind 1: binary64 Q."""
    _anonymous_ = ("u",)
    _fields_ = [("q_hash", ctypes.c_uint64), ("n", ctypes.c_int32), ("split_bits", ctypes.c_int32),
                ("prefix_bits", ctypes.c_int32), ("chunk_bits", ctypes.c_int32),
                ("sub", ctypes.c_uint64), ("next", ctypes.c_uint64),
                ("steps_done", ctypes.c_uint64), ("steps_total", ctypes.c_uint64),
                ("done", ctypes.c_int32), ("have_best", ctypes.c_int32), ("u", _Best),
                ("kind", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]

    def result(self) -> "Result":
        if not self.have_best:
            raise ValueError("no state searched yet")
        b = self.best_f64 if self.kind == 1 else self.best
        return Result(b.min_energy, b.argmin, b.count)


class ProgressLowest(ctypes.Structure):
    """The state of a spectrum run in slices (``qubo_progress_lowest``, 1128
    bytes): the run's header (kind 2) and the k lowest states found so far."""
    _fields_ = [("head", Progress), ("k", ctypes.c_int32), ("found", ctypes.c_int32),
                ("states", _State * 64)]

    @property
    def done(self) -> bool:
        return bool(self.head.done)

    def result(self) -> list[tuple[int, int]]:
        return [(self.states[i].energy, self.states[i].index) for i in range(self.found)]


class _Timing(ctypes.Structure):
    _fields_ = [("build_ms", ctypes.c_float), ("search_ms", ctypes.c_float),
                ("reduce_ms", ctypes.c_float), ("total_ms", ctypes.c_float),
                ("states", ctypes.c_uint64), ("blocks", ctypes.c_int32), ("cols_per_lane", ctypes.c_uint32),
                ("bodies", ctypes.c_uint64), ("checked_bodies", ctypes.c_uint64),
                ("slow_bodies", ctypes.c_uint64), ("candidates", ctypes.c_uint64)]


@dataclass(frozen=True)
class Result:
    min_energy: int
    argmin: int
    count: int

    def triple(self) -> tuple[int, int, int]:
        return (self.min_energy, self.argmin, self.count)

    def bits(self, n: int) -> list[int]:
        """The minimiser as a 0/1 list, variable 0 first."""
        return [(self.argmin >> (n - 1 - i)) & 1 for i in range(n)]


_lib = None

EXPORTS = ("qubo_make_plan", "qubo_check_q", "qubo_abs_sum", "qubo_check_q_f64", "qubo_f64_as_int32", "qubo_search", "qubo_search_noalloc", "qubo_search_range", "qubo_search_ex",
           "qubo_build_tables", "qubo_last_timing", "qubo_search_lowest", "qubo_search_f64",
           "qubo_search_lowest_f64",
           "qubo_progress_init", "qubo_search_step", "qubo_progress_init_lowest", "qubo_search_step_lowest",
           "qubo_progress_init_f64", "qubo_search_step_f64", "qubo_strerror", "qubo_version")
MAX_LOWEST = 64
FLAG_STRICT_MIN = 1
FLAG_COLS8 = 2
FLAG_COLS16 = 4
FLAG_SPLIT_SHIFT = 8


def load(path: str = LIB_PATH):
    """Loads libqubo.so (built by ``python -m ising_ground_state_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libqubo.so not built: run `python -m ising_ground_state_amd.build` "
                           "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(path)
    i32p = ctypes.c_void_p
    lib.qubo_make_plan.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(_Plan)]
    lib.qubo_check_q.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.qubo_abs_sum.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64)]
    lib.qubo_check_q_f64.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.qubo_f64_as_int32.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
    lib.qubo_search.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                ctypes.POINTER(_Result)]
    lib.qubo_search_noalloc.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.POINTER(_Result)]
    lib.qubo_search_range.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                      ctypes.c_uint64, ctypes.c_void_p, ctypes.POINTER(_Result)]
    lib.qubo_search_ex.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                   ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.POINTER(_Result)]
    lib.qubo_build_tables.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]
    lib.qubo_last_timing.argtypes = [ctypes.POINTER(_Timing)]
    lib.qubo_search_lowest.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p,
                                       ctypes.POINTER(_State), ctypes.POINTER(ctypes.c_int)]
    lib.qubo_strerror.argtypes = [ctypes.c_int]
    lib.qubo_strerror.restype = ctypes.c_char_p
    lib.qubo_version.restype = ctypes.c_char_p
    lib.qubo_search_f64.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                    ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.POINTER(_ResultF64)]
    lib.qubo_progress_init.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                                       ctypes.c_void_p, ctypes.POINTER(Progress)]
    lib.qubo_search_step.argtypes = [i32p, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(Progress)]
    lib.qubo_search_lowest_f64.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32,
                                           ctypes.c_void_p, ctypes.POINTER(_StateF64),
                                           ctypes.POINTER(ctypes.c_int)]
    lib.qubo_progress_init_lowest.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_uint32, ctypes.c_void_p, ctypes.POINTER(ProgressLowest)]
    lib.qubo_search_step_lowest.argtypes = [i32p, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ProgressLowest)]
    lib.qubo_progress_init_f64.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.POINTER(Progress)]
    lib.qubo_search_step_f64.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(Progress)]
    for name in EXPORTS:
        if name not in ("qubo_strerror", "qubo_version"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().qubo_strerror(code).decode()


def version() -> str:
    return load().qubo_version().decode()


def _opt(v) -> int:
    return -1 if v is None else int(v)


def make_plan(n: int, prefix_bits: int | None = None, cache_bits: int | None = None) -> dict:
    """Host-only plan of a search of n variables (no device needed), for the
    default kernel build."""
    p = _Plan()
    rc = load().qubo_make_plan(int(n), _opt(prefix_bits), _opt(cache_bits), ctypes.byref(p))
    if rc != QUBO_OK:
        raise QuboError(rc, "qubo_make_plan")
    return {name: getattr(p, name) for name, _ in _Plan._fields_}


def check_q(Q_host) -> int:
    """Host-only overflow guard on a host int32 matrix; returns sum |Q_ij|."""
    import numpy as np
    q = np.ascontiguousarray(np.asarray(Q_host, dtype=np.int32))
    if q.ndim != 2 or q.shape[0] != q.shape[1]:
        raise ValueError("Q must be square")
    lib = load()
    rc = lib.qubo_check_q(q.ctypes.data_as(ctypes.c_void_p), q.shape[0])
    if rc != QUBO_OK:
        raise QuboError(rc, "qubo_check_q")
    s = ctypes.c_int64(0)
    rc = lib.qubo_abs_sum(q.ctypes.data_as(ctypes.c_void_p), q.shape[0], ctypes.byref(s))
    if rc != QUBO_OK:
        raise QuboError(rc, "qubo_abs_sum")
    return int(s.value)


def check_q_f64(Q_host) -> None:
    """Host-only guard of the binary64 searches on a host matrix (raises
    QuboError(QUBO_ERANGE) for a non-finite entry or sum |Q_ij| outside
    {0} and [2^-100, 2^100])."""
    import numpy as np
    q = np.ascontiguousarray(np.asarray(Q_host, dtype=np.float64))
    if q.ndim != 2 or q.shape[0] != q.shape[1]:
        raise ValueError("Q must be square")
    rc = load().qubo_check_q_f64(q.ctypes.data_as(ctypes.c_void_p), q.shape[0])
    if rc != QUBO_OK:
        raise QuboError(rc, "qubo_check_q_f64")


def f64_as_int32(Q_host):
    """The exact int32 form of a dyadic binary64 host matrix: (Q_int, f) with
    Q = Q_int / 2^f entry by entry and sum |Q_int| <= 2^30 - 1, the form the
    binary64 searches hand to the integer search.  Raises QuboError(QUBO_ERANGE)
    when Q has no such form."""
    import numpy as np
    q = np.ascontiguousarray(np.asarray(Q_host, dtype=np.float64))
    if q.ndim != 2 or q.shape[0] != q.shape[1]:
        raise ValueError("Q must be square")
    out = np.zeros(q.shape, dtype=np.int32)
    f = ctypes.c_int(0)
    rc = load().qubo_f64_as_int32(q.ctypes.data_as(ctypes.c_void_p), q.shape[0],
                                  out.ctypes.data_as(ctypes.c_void_p), ctypes.byref(f))
    if rc != QUBO_OK:
        raise QuboError(rc, "qubo_f64_as_int32")
    return out, f.value


def _device_q(Q):
    import torch
    if not isinstance(Q, torch.Tensor) or not Q.is_cuda:
        raise TypeError("Q must be a torch tensor on a HIP device")
    if Q.dtype != torch.int32:
        raise TypeError("Q must be int32")
    if Q.dim() != 2 or Q.shape[0] != Q.shape[1]:
        raise ValueError("Q must be square")
    return Q.contiguous()


def _stream(Q, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(Q.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _flags(strict: bool, cols_per_lane: int | None, split_bits: int | None = None) -> int:
    f = FLAG_STRICT_MIN if strict else 0
    if cols_per_lane is not None:
        f |= {8: FLAG_COLS8, 16: FLAG_COLS16}[int(cols_per_lane)]
    if split_bits:
        if not 0 < int(split_bits) < 64:
            raise ValueError("split_bits must be in 1..63")
        f |= int(split_bits) << FLAG_SPLIT_SHIFT
    return f


def search(Q, prefix_bits: int | None = None, cache_bits: int | None = None, stream=None,
           strict: bool = False, cols_per_lane: int | None = None, split_bits: int | None = None) -> Result:
    """Exhaustive search of min_x x^T Q x over {0,1}^n on Q's device.

    strict=True takes the minimum after every prefix (Algorithm 2 as printed)
    instead of gating it by the per-block lower bound; cols_per_lane (8 or 16)
    picks the kernel build; split_bits=k searches the 2^k sub-problems with the
    first k variables fixed, one launch each (automatic above 58 variables).
    The result never depends on these options."""
    import torch
    Q = _device_q(Q)
    r = _Result()
    flags = _flags(strict, cols_per_lane, split_bits)
    with torch.cuda.device(Q.device):
        if flags:
            rc = load().qubo_search_ex(ctypes.c_void_p(Q.data_ptr()), Q.shape[0], _opt(prefix_bits),
                                       _opt(cache_bits), 0, 0, flags, _stream(Q, stream),
                                       ctypes.byref(r))
        else:
            rc = load().qubo_search(ctypes.c_void_p(Q.data_ptr()), Q.shape[0], _opt(prefix_bits),
                                    _opt(cache_bits), _stream(Q, stream), ctypes.byref(r))
    if rc != QUBO_OK:
        raise QuboError(rc, "qubo_search")
    return Result(r.min_energy, r.argmin, r.count)


def search_noalloc(Q, prefix_bits: int | None = None, cache_bits: int | None = None, stream=None) -> Result:
    """search() through qubo_search_noalloc: no device allocation; the library's
    static 128 MiB buffer per GPU holds the workspace (QuboError(QUBO_ESCRATCH)
    when the plan needs more).  Calls that overlap on one GPU must be
    serialised."""
    import torch
    Q = _device_q(Q)
    r = _Result()
    with torch.cuda.device(Q.device):
        rc = load().qubo_search_noalloc(ctypes.c_void_p(Q.data_ptr()), Q.shape[0], _opt(prefix_bits),
                                        _opt(cache_bits), _stream(Q, stream), ctypes.byref(r))
    if rc != QUBO_OK:
        raise QuboError(rc, "qubo_search_noalloc")
    return Result(r.min_energy, r.argmin, r.count)


def search_range(Q, prefix_bits: int, gray_lo: int, gray_hi: int, cache_bits: int | None = None,
                 stream=None, strict: bool = False, cols_per_lane: int | None = None) -> Result:
    """Search the prefixes g(j), gray_lo <= j < gray_hi, with every suffix."""
    import torch
    Q = _device_q(Q)
    r = _Result()
    with torch.cuda.device(Q.device):
        rc = load().qubo_search_ex(ctypes.c_void_p(Q.data_ptr()), Q.shape[0], int(prefix_bits),
                                   _opt(cache_bits), int(gray_lo), int(gray_hi),
                                   _flags(strict, cols_per_lane), _stream(Q, stream), ctypes.byref(r))
    if rc != QUBO_OK:
        raise QuboError(rc, "qubo_search_range")
    return Result(r.min_energy, r.argmin, r.count)


def lowest(Q, k: int, prefix_bits: int | None = None, cache_bits: int | None = None, stream=None,
           cols_per_lane: int | None = None, split_bits: int | None = None, gray_lo: int = 0,
           gray_hi: int = 0) -> list[tuple[int, int]]:
    """The k lowest states (k <= 64) as (energy, index) pairs, energy ascending
    then index ascending: the low-energy spectrum.  gray_lo/gray_hi select a
    slice as in search_range (prefix_bits must then be given).  A float64 Q
    gives binary64 energies (search_f64's definition; no outer split)."""
    import torch
    if _is_f64(Q):
        if split_bits or (cols_per_lane not in (None, 8)):
            raise ValueError("the binary64 spectrum has no outer split and 8 columns per lane")
        Q = _device_f64(Q)
        k = int(k)
        outf = (_StateF64 * max(k, 1))()
        found = ctypes.c_int(0)
        with torch.cuda.device(Q.device):
            rc = load().qubo_search_lowest_f64(ctypes.c_void_p(Q.data_ptr()), Q.shape[0], k, _opt(prefix_bits),
                                               _opt(cache_bits), int(gray_lo), int(gray_hi), 0,
                                               _stream(Q, stream), outf, ctypes.byref(found))
        if rc != QUBO_OK:
            raise QuboError(rc, "qubo_search_lowest_f64")
        return [(outf[i].energy, outf[i].index) for i in range(found.value)]
    Q = _device_q(Q)
    k = int(k)
    out = (_State * max(k, 1))()
    found = ctypes.c_int(0)
    with torch.cuda.device(Q.device):
        rc = load().qubo_search_lowest(ctypes.c_void_p(Q.data_ptr()), Q.shape[0], k, _opt(prefix_bits),
                                       _opt(cache_bits), int(gray_lo), int(gray_hi),
                                       _flags(False, cols_per_lane, split_bits), _stream(Q, stream),
                                       out, ctypes.byref(found))
    if rc != QUBO_OK:
        raise QuboError(rc, "qubo_search_lowest")
    return [(out[i].energy, out[i].index) for i in range(found.value)]


def _is_f64(Q) -> bool:
    import torch
    return isinstance(Q, torch.Tensor) and Q.dtype == torch.float64


def _device_f64(Q):
    import torch
    if not isinstance(Q, torch.Tensor) or not Q.is_cuda or Q.dtype != torch.float64:
        raise TypeError("Q must be a float64 torch tensor on a HIP device")
    if Q.dim() != 2 or Q.shape[0] != Q.shape[1]:
        raise ValueError("Q must be square")
    return Q.contiguous()


def progress_init(Q, prefix_bits: int | None = None, chunk_bits: int | None = None,
                  split_bits: int | None = None, stream=None, k: int | None = None):
    """Starts a search run in slices of 2^chunk_bits Gray steps (default: about
    2^48 states per step); split_bits as for search.  An int32 Q runs
    qubo_search's definition (with k: qubo_search_lowest's k lowest states,
    returning a ProgressLowest), a float64 Q qubo_search_f64's (no split)."""
    import torch
    if k is not None:
        Q = _device_q(Q)
        pl = ProgressLowest()
        with torch.cuda.device(Q.device):
            rc = load().qubo_progress_init_lowest(ctypes.c_void_p(Q.data_ptr()), Q.shape[0], int(k),
                                                  _opt(prefix_bits), _opt(chunk_bits),
                                                  _flags(False, None, split_bits), _stream(Q, stream),
                                                  ctypes.byref(pl))
        if rc != QUBO_OK:
            raise QuboError(rc, "qubo_progress_init_lowest")
        return pl
    p = Progress()
    if _is_f64(Q):
        if split_bits:
            raise ValueError("a binary64 run has no outer split")
        Q = _device_f64(Q)
        with torch.cuda.device(Q.device):
            rc = load().qubo_progress_init_f64(ctypes.c_void_p(Q.data_ptr()), Q.shape[0], _opt(prefix_bits),
                                               _opt(chunk_bits), _stream(Q, stream), ctypes.byref(p))
        if rc != QUBO_OK:
            raise QuboError(rc, "qubo_progress_init_f64")
        return p
    Q = _device_q(Q)
    with torch.cuda.device(Q.device):
        rc = load().qubo_progress_init(ctypes.c_void_p(Q.data_ptr()), Q.shape[0], _opt(prefix_bits),
                                       _opt(chunk_bits), _flags(False, None, split_bits), _stream(Q, stream),
                                       ctypes.byref(p))
    if rc != QUBO_OK:
        raise QuboError(rc, "qubo_progress_init")
    return p


def search_step(Q, progress, stream=None) -> bool:
    """Searches the next slice of the run and updates ``progress`` (a Progress
    or a ProgressLowest) in place; returns whether the run is done."""
    import torch
    f64 = _is_f64(Q)
    Q = _device_f64(Q) if f64 else _device_q(Q)
    if isinstance(progress, ProgressLowest):
        name = "qubo_search_step_lowest"
    else:
        name = "qubo_search_step_f64" if f64 else "qubo_search_step"
    with torch.cuda.device(Q.device):
        rc = getattr(load(), name)(ctypes.c_void_p(Q.data_ptr()), Q.shape[0], _stream(Q, stream),
                                   ctypes.byref(progress))
    if rc != QUBO_OK:
        raise QuboError(rc, name)
    return bool(progress.done)


def search_resumable(Q, path: str, prefix_bits: int | None = None, chunk_bits: int | None = None,
                     split_bits: int | None = None, max_steps: int | None = None, stream=None,
                     k: int | None = None):
    """A search that survives interruption: the run's state (96 bytes; 1128 for
    a spectrum run, k given) is kept in the file ``path`` and rewritten
    atomically after every step, and a later call with the same Q continues
    from it.  Q is int32 or float64 (as for search and search_f64).  Returns the
    Result (the k lowest states for a spectrum run) once every state has been
    searched, or None after max_steps steps of an unfinished run."""
    kind = ProgressLowest if k is not None else Progress
    if os.path.exists(path):
        with open(path, "rb") as f:
            raw = f.read()
        if len(raw) != ctypes.sizeof(kind):
            raise ValueError("%s is not a search state of this kind (%d bytes)" % (path, len(raw)))
        p = kind.from_buffer_copy(raw)
    else:
        p = progress_init(Q, prefix_bits, chunk_bits, split_bits, stream, k=k)
        _save_progress(path, p)
    steps = 0
    while not p.done and (max_steps is None or steps < max_steps):
        search_step(Q, p, stream)
        _save_progress(path, p)
        steps += 1
    return p.result() if p.done else None


def _save_progress(path: str, p) -> None:
    tmp = path + ".tmp"
    with open(tmp, "wb") as f:
        f.write(bytes(p))
        f.flush()
        os.fsync(f.fileno())
    os.replace(tmp, path)


def search_f64(Q, prefix_bits: int | None = None, cache_bits: int | None = None, stream=None,
               gray_lo: int = 0, gray_hi: int = 0) -> Result:
    """Exhaustive search of a real-valued (float64) Q: the minimum of the
    binary64 energy summed in row-major order over the set variables, its
    lowest minimiser and the exact count.  Returns a Result with a float
    min_energy."""
    import torch
    if not isinstance(Q, torch.Tensor) or not Q.is_cuda or Q.dtype != torch.float64:
        raise TypeError("Q must be a float64 torch tensor on a HIP device")
    if Q.dim() != 2 or Q.shape[0] != Q.shape[1]:
        raise ValueError("Q must be square")
    Q = Q.contiguous()
    r = _ResultF64()
    with torch.cuda.device(Q.device):
        rc = load().qubo_search_f64(ctypes.c_void_p(Q.data_ptr()), Q.shape[0], _opt(prefix_bits),
                                    _opt(cache_bits), int(gray_lo), int(gray_hi), 0, _stream(Q, stream),
                                    ctypes.byref(r))
    if rc != QUBO_OK:
        raise QuboError(rc, "qubo_search_f64")
    return Result(r.min_energy, r.argmin, r.count)


def build_tables(Q, prefix_bits: int, stream=None):
    """The cache tables (E_s, M_int, Gray-ordered E_p) as int32 device tensors."""
    import torch
    Q = _device_q(Q)
    n = Q.shape[0]
    A, B = int(prefix_bits), n - int(prefix_bits)
    es = torch.empty(1 << B, dtype=torch.int32, device=Q.device)
    mint = torch.empty((A, 1 << B), dtype=torch.int32, device=Q.device)
    ep = torch.empty(1 << A, dtype=torch.int32, device=Q.device)
    with torch.cuda.device(Q.device):
        rc = load().qubo_build_tables(ctypes.c_void_p(Q.data_ptr()), n, A, ctypes.c_void_p(es.data_ptr()),
                                      ctypes.c_void_p(mint.data_ptr()), ctypes.c_void_p(ep.data_ptr()),
                                      _stream(Q, stream))
    if rc != QUBO_OK:
        raise QuboError(rc, "qubo_build_tables")
    return es, mint, ep


def last_timing() -> dict:
    """Device times (ms) of the last search on this thread, from HIP events on its stream."""
    t = _Timing()
    load().qubo_last_timing(ctypes.byref(t))
    return {name: getattr(t, name) for name, _ in _Timing._fields_}
