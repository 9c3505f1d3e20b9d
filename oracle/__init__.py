"""CPU oracle for band -> bidiagonal bulge chasing.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``band_bidiagonal_bulge_amd``); the two meet only through the seeded input
generators in ``bb_inputs``.

The arithmetic lives in ``bb_oracle.c`` / ``bb_oracle_body.h`` (plain C, one
scalar loop per step of the method, fp32 or fp64).  This module builds that
library with gcc and marshals numpy arrays to it.

Follows the page "Accelerating Bidiagonalization of Banded Matrices through
Memory-Aware Bulge-Chasing on GPUs" (three-cycle-separation passage,
Algorithm 2 passage) and the page "A two-stage reduction on an Apple M5 Pro",
section 6 (one row or one column cleared per reflector, sweeps chasing their
bulge a block of b at a time).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = [os.path.join(_HERE, "bb_oracle.c"), os.path.join(_HERE, "bb_oracle_body.h")]
_LIB_PATH = os.path.join(_HERE, "libbb_oracle.so")
# -ffp-contract=off: only the explicit fma() calls fuse; -mfma lets gcc emit
# them as single instructions (correctly rounded either way).
_CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-mfma", "-fno-math-errno"]

_MT_SRC = [os.path.join(_HERE, "bb_oracle_mt.c"), os.path.join(_HERE, "bb_oracle_mt_body.h")] + _SRC
_MT_LIB_PATH = os.path.join(_HERE, "libbb_oracle_mt.so")

_SV_SRC = [os.path.join(_HERE, "bb_oracle_svals.c"), os.path.join(_HERE, "bb_oracle_svals_body.h")]
_SV_LIB_PATH = os.path.join(_HERE, "libbb_oracle_svals.so")

_SYM_SRC = [os.path.join(_HERE, "bb_oracle_sym.c"), os.path.join(_HERE, "bb_oracle_sym_body.h")]
_SYM_LIB_PATH = os.path.join(_HERE, "libbb_oracle_sym.so")

_F16_SRC = [os.path.join(_HERE, "bb_oracle_f16.cpp")] + _SRC
_F16_LIB_PATH = os.path.join(_HERE, "libbb_oracle_f16.so")

_lib = None
_mt_lib = None
_sv_lib = None
_sym_lib = None
_f16_lib = None


def build_f16(force: bool = False) -> str:
    """Compile the fp16 oracle (the same body on an emulated binary16 type)."""
    stale = not os.path.exists(_F16_LIB_PATH) or any(
        os.path.getmtime(s) > os.path.getmtime(_F16_LIB_PATH) for s in _F16_SRC)
    if force or stale:
        tmp = _F16_LIB_PATH + ".tmp%d" % os.getpid()
        flags = [f for f in _CFLAGS if f != "-std=c99"]
        cmd = ["g++", *flags, "-std=c++17", "-o", tmp, _F16_SRC[0], "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _F16_LIB_PATH)
    return _F16_LIB_PATH


def f16_lib():
    global _f16_lib
    if _f16_lib is None:
        if not _cpu_has_fma():
            raise RuntimeError("oracle build uses the FMA instruction; this host CPU lacks it")
        path = _F16_LIB_PATH if os.path.exists(_F16_LIB_PATH) else build_f16()
        L = ctypes.CDLL(path)
        i64, i32, vp, u16 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_uint16
        L.bb_oracle_reduce_f16.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, i64, ctypes.POINTER(i64)]
        L.bb_oracle_reduce_f16.restype = i32
        L.bb_oracle_h16_from_double.argtypes = [ctypes.c_double]
        L.bb_oracle_h16_from_double.restype = u16
        L.bb_oracle_h16_to_double.argtypes = [u16]
        L.bb_oracle_h16_to_double.restype = ctypes.c_double
        for f in ("bb_oracle_h16_fma",):
            getattr(L, f).argtypes = [u16, u16, u16]
            getattr(L, f).restype = u16
        for f in ("bb_oracle_h16_div",):
            getattr(L, f).argtypes = [u16, u16]
            getattr(L, f).restype = u16
        L.bb_oracle_h16_sqrt.argtypes = [u16]
        L.bb_oracle_h16_sqrt.restype = u16
        _f16_lib = L
    return _f16_lib


def build_sym(force: bool = False) -> str:
    """Compile the symmetric band -> tridiagonal oracle."""
    stale = not os.path.exists(_SYM_LIB_PATH) or any(
        os.path.getmtime(s) > os.path.getmtime(_SYM_LIB_PATH) for s in _SYM_SRC)
    if force or stale:
        tmp = _SYM_LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", *_CFLAGS, "-o", tmp, _SYM_SRC[0], "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SYM_LIB_PATH)
    return _SYM_LIB_PATH


def sym_lib():
    global _sym_lib
    if _sym_lib is None:
        if not _cpu_has_fma():
            raise RuntimeError("oracle build uses the FMA instruction; this host CPU lacks it")
        path = _SYM_LIB_PATH if os.path.exists(_SYM_LIB_PATH) else build_sym()
        L = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        for suf in ("f64", "f32"):
            f = getattr(L, "bb_oracle_sym_reduce_" + suf)
            f.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp]
            f.restype = i32
            g = getattr(L, "bb_oracle_sym_run_cycles_" + suf)
            g.argtypes = [vp, i64, i64, i32, i32, vp, i64, vp]
            g.restype = i32
        L.bb_oracle_sym_ld.argtypes = [i64, i32, i32]
        L.bb_oracle_sym_ld.restype = i64
        _sym_lib = L
    return _sym_lib


def build_svals(force: bool = False) -> str:
    """Compile the bisection oracle (bidiagonal -> singular values)."""
    stale = not os.path.exists(_SV_LIB_PATH) or any(
        os.path.getmtime(s) > os.path.getmtime(_SV_LIB_PATH) for s in _SV_SRC)
    if force or stale:
        tmp = _SV_LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", *_CFLAGS, "-o", tmp, _SV_SRC[0], "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SV_LIB_PATH)
    return _SV_LIB_PATH


def svals_lib():
    global _sv_lib
    if _sv_lib is None:
        path = _SV_LIB_PATH if os.path.exists(_SV_LIB_PATH) else build_svals()
        L = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        for suf, real in (("f64", ctypes.c_double), ("f32", ctypes.c_float)):
            f = getattr(L, "bb_oracle_svals_" + suf)
            f.argtypes = [vp, vp, i64, i64, i64, vp]
            f.restype = ctypes.c_int
            g = getattr(L, "bb_oracle_gk_count_" + suf)
            g.argtypes = [vp, vp, i64, real, real]
            g.restype = i64
            h = getattr(L, "bb_oracle_gk_interval_" + suf)
            h.argtypes = [vp, vp, i64, vp, vp, vp]
            h.restype = None
        _sv_lib = L
    return _sv_lib


def build_mt(force: bool = False) -> str:
    """Compile the threaded runner (the oracle's cycles on host threads)."""
    stale = not os.path.exists(_MT_LIB_PATH) or any(
        os.path.getmtime(s) > os.path.getmtime(_MT_LIB_PATH) for s in _MT_SRC)
    if force or stale:
        tmp = _MT_LIB_PATH + ".tmp%d" % os.getpid()
        flags = [f if f != "-std=c99" else "-std=c11" for f in _CFLAGS]
        cmd = ["gcc", *flags, "-pthread", "-o", tmp, _MT_SRC[0], "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _MT_LIB_PATH)
    return _MT_LIB_PATH


def mt_lib():
    global _mt_lib
    if _mt_lib is None:
        if not _cpu_has_fma():
            raise RuntimeError("oracle build uses the FMA instruction; this host CPU lacks it")
        path = _MT_LIB_PATH if os.path.exists(_MT_LIB_PATH) else build_mt()
        L = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        for suf in ("f64", "f32"):
            f = getattr(L, "bb_oracle_mt_reduce_" + suf)
            f.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, i32, i32, ctypes.POINTER(i32)]
            f.restype = i32
        L.bb_oracle_mt_default_threads.restype = i32
        _mt_lib = L
    return _mt_lib


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (host only).  Returns the library path."""
    stale = not os.path.exists(_LIB_PATH) or any(
        os.path.getmtime(s) > os.path.getmtime(_LIB_PATH) for s in _SRC)
    if force or stale:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", *_CFLAGS, "-o", tmp, _SRC[0], "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _cpu_has_fma() -> bool:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("flags"):
                    return " fma " in (line.rstrip() + " ")
    except OSError:
        pass
    return True


def lib():
    global _lib
    if _lib is None:
        if not _cpu_has_fma():
            raise RuntimeError("oracle build uses the FMA instruction; this host CPU lacks it")
        path = _LIB_PATH if os.path.exists(_LIB_PATH) else build()
        L = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        for suf in ("f64", "f32"):
            f = getattr(L, "bb_oracle_reduce_" + suf)
            f.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp, i64, ctypes.POINTER(i64)]
            f.restype = i32
            g = getattr(L, "bb_oracle_run_cycles_" + suf)
            g.argtypes = [vp, i64, i64, i32, i32, vp, i64, vp]
            g.restype = i32
        L.bb_oracle_ld.argtypes = [i64, i32, i32]
        L.bb_oracle_ld.restype = i64
        L.bb_oracle_T.argtypes = [i64, i32, i32]
        L.bb_oracle_T.restype = i64
        _lib = L
    return _lib


def _np_dtype(name):
    return {"f16": np.float16, "f32": np.float32, "f64": np.float64}[name]


def _suffix(dt):
    return {np.dtype(np.float16): "f16", np.dtype(np.float32): "f32"}.get(np.dtype(dt), "f64")


def working_ld(n: int, bw: int, tw: int) -> int:
    """Stored diagonals of the working band: T sub + diagonal + BW+T super."""
    return int(lib().bb_oracle_ld(n, bw, tw))


def working_T(n: int, bw: int, tw: int) -> int:
    return int(lib().bb_oracle_T(n, bw, tw))


def reduce(band: np.ndarray, bw: int, tw: int, compute: str | None = None,
           return_band: bool = False, max_cycles: int = -1):
    """Sequential bulge-chasing reduction of an upper band.

    band     (n, >= bw+1) array, row i holds A(i, i..i+bw); entries past n
             are ignored.  Its dtype (f16/f32/f64) is the storage precision.
    compute  'f16', 'f32' or 'f64' (default: the band's dtype).  A band of
             lower precision is widened exactly before the reduction.
    Returns (d, e) or (d, e, working_band, T) with return_band.
    With max_cycles >= 0 the reduction stops early (bench sampling only) and
    the third return value is the number of cycles executed.
    """
    band = np.asarray(band)
    n = band.shape[0]
    cdt = _np_dtype(compute) if compute else band.dtype
    a = np.ascontiguousarray(band, dtype=cdt)
    d = np.zeros(n, dtype=cdt)
    e = np.zeros(max(n - 1, 0), dtype=cdt)
    ld = working_ld(n, bw, tw)
    out = np.zeros((n, ld), dtype=cdt) if return_band else None
    done = ctypes.c_int64(0)
    suf = _suffix(cdt)
    f = getattr(f16_lib() if suf == "f16" else lib(), "bb_oracle_reduce_" + suf)
    rc = f(a.ctypes.data, a.shape[1], n, bw, tw, d.ctypes.data,
           e.ctypes.data if e.size else None,
           out.ctypes.data if out is not None else None, max_cycles, ctypes.byref(done))
    if rc != 0:
        raise ValueError("oracle rejected arguments (rc=%d)" % rc)
    if max_cycles >= 0:
        return d, e, int(done.value)
    if return_band:
        return d, e, out, working_T(n, bw, tw)
    return d, e


def run_cycles(band: np.ndarray, bw: int, tw: int, order, compute: str | None = None):
    """Runs the given (pass, R, k) cycles in order; returns the working band."""
    band = np.asarray(band)
    n = band.shape[0]
    cdt = _np_dtype(compute) if compute else band.dtype
    a = np.ascontiguousarray(band, dtype=cdt)
    o = np.ascontiguousarray(np.asarray(order, dtype=np.int32).reshape(-1, 3))
    out = np.zeros((n, working_ld(n, bw, tw)), dtype=cdt)
    f = getattr(lib(), "bb_oracle_run_cycles_" + _suffix(cdt))
    rc = f(a.ctypes.data, a.shape[1], n, bw, tw, o.ctypes.data, o.shape[0], out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected the cycle list (rc=%d)" % rc)
    return out


def band_to_dense(work: np.ndarray, T: int) -> np.ndarray:
    """Dense n x n matrix from a working band (element (i,j) at [i, j-i+T])."""
    n, ld = work.shape
    A = np.zeros((n, n), dtype=work.dtype)
    for i in range(n):
        for o in range(ld):
            j = i + o - T
            if 0 <= j < n:
                A[i, j] = work[i, o]
    return A


def reduce_mt(band: np.ndarray, bw: int, tw: int, threads: int = 0, compute: str | None = None,
              return_band: bool = False, max_passes: int = -1):
    """The oracle's reduction with each pass's sweeps on host threads;
    bitwise equal to :func:`reduce`.  threads > 0: exactly that many (at most
    one per sweep); threads < 0: at most -threads, capped per pass at 2n/(3b)
    and n/256 (page "A two-stage reduction on an Apple M5 Pro", section 6);
    0: every online core, capped the same way.  max_passes >= 0 stops
    after that many passes (timing samples).  Returns (d, e, threads_used) or,
    with return_band, (d, e, working_band, T, threads_used)."""
    band = np.asarray(band)
    n = band.shape[0]
    cdt = _np_dtype(compute) if compute else band.dtype
    a = np.ascontiguousarray(band, dtype=cdt)
    d = np.zeros(n, dtype=cdt)
    e = np.zeros(max(n - 1, 0), dtype=cdt)
    out = np.zeros((n, working_ld(n, bw, tw)), dtype=cdt) if return_band else None
    used = ctypes.c_int(0)
    f = getattr(mt_lib(), "bb_oracle_mt_reduce_" + _suffix(cdt))
    rc = f(a.ctypes.data, a.shape[1], n, bw, tw, d.ctypes.data, e.ctypes.data if e.size else None,
           out.ctypes.data if out is not None else None, threads, max_passes, ctypes.byref(used))
    if rc != 0:
        raise ValueError("threaded oracle rejected arguments (rc=%d)" % rc)
    if return_band:
        return d, e, out, working_T(n, bw, tw), int(used.value)
    return d, e, int(used.value)


def _bidiag_args(d, e):
    d = np.ascontiguousarray(d)
    if d.dtype not in (np.float32, np.float64):
        raise ValueError("d must be float32 or float64")
    e = np.ascontiguousarray(e, dtype=d.dtype)
    if e.size != max(d.size - 1, 0):
        raise ValueError("e must have n-1 entries")
    return d, e


def svals(d: np.ndarray, e: np.ndarray, i0: int = 0, i1: int | None = None) -> np.ndarray:
    """Singular values i0..i1-1 (descending) of the upper bidiagonal (d, e),
    by bisection on the Golub-Kahan tridiagonal in the precision of d."""
    d, e = _bidiag_args(d, e)
    n = d.size
    i1 = n if i1 is None else i1
    out = np.zeros(max(i1 - i0, 0), dtype=d.dtype)
    f = getattr(svals_lib(), "bb_oracle_svals_" + _suffix(d.dtype))
    rc = f(d.ctypes.data, e.ctypes.data if e.size else None, n, i0, i1, out.ctypes.data)
    if rc != 0:
        raise ValueError("bisection oracle rejected arguments (rc=%d)" % rc)
    return out


def gk_interval(d: np.ndarray, e: np.ndarray):
    """(lo, hi, pivmin) of the Golub-Kahan tridiagonal of (d, e)."""
    d, e = _bidiag_args(d, e)
    lo, hi, pm = (np.zeros(1, dtype=d.dtype) for _ in range(3))
    getattr(svals_lib(), "bb_oracle_gk_interval_" + _suffix(d.dtype))(
        d.ctypes.data, e.ctypes.data if e.size else None, d.size, lo.ctypes.data, hi.ctypes.data,
        pm.ctypes.data)
    return lo[0], hi[0], pm[0]


def gk_count(d: np.ndarray, e: np.ndarray, x: float, pivmin: float) -> int:
    """Sturm count: eigenvalues of the Golub-Kahan tridiagonal <= x."""
    d, e = _bidiag_args(d, e)
    f = getattr(svals_lib(), "bb_oracle_gk_count_" + _suffix(d.dtype))
    return int(f(d.ctypes.data, e.ctypes.data if e.size else None, d.size, x, pivmin))


def sym_working_ld(n: int, bw: int, tw: int) -> int:
    """Stored superdiagonals of the symmetric working band (BW + T + 1)."""
    return int(sym_lib().bb_oracle_sym_ld(n, bw, tw))


def sym_reduce(band: np.ndarray, bw: int, tw: int, compute: str | None = None, return_band: bool = False):
    """Symmetric band -> tridiagonal.  band: (n, >= bw+1), row i holds
    A(i, i..i+bw) = A(i..i+bw, i).  Returns (d, e) or (d, e, working_band)."""
    band = np.asarray(band)
    n = band.shape[0]
    cdt = _np_dtype(compute) if compute else band.dtype
    a = np.ascontiguousarray(band, dtype=cdt)
    d = np.zeros(n, dtype=cdt)
    e = np.zeros(max(n - 1, 0), dtype=cdt)
    out = np.zeros((n, sym_working_ld(n, bw, tw)), dtype=cdt) if return_band else None
    f = getattr(sym_lib(), "bb_oracle_sym_reduce_" + _suffix(cdt))
    rc = f(a.ctypes.data, a.shape[1], n, bw, tw, d.ctypes.data, e.ctypes.data if e.size else None,
           out.ctypes.data if out is not None else None)
    if rc != 0:
        raise ValueError("symmetric oracle rejected arguments (rc=%d)" % rc)
    return (d, e, out) if return_band else (d, e)


def sym_run_cycles(band: np.ndarray, bw: int, tw: int, order, compute: str | None = None):
    """Runs the given (pass, R, k) cycles in order; returns the working band."""
    band = np.asarray(band)
    n = band.shape[0]
    cdt = _np_dtype(compute) if compute else band.dtype
    a = np.ascontiguousarray(band, dtype=cdt)
    o = np.ascontiguousarray(np.asarray(order, dtype=np.int32).reshape(-1, 3))
    out = np.zeros((n, sym_working_ld(n, bw, tw)), dtype=cdt)
    f = getattr(sym_lib(), "bb_oracle_sym_run_cycles_" + _suffix(cdt))
    rc = f(a.ctypes.data, a.shape[1], n, bw, tw, o.ctypes.data, o.shape[0], out.ctypes.data)
    if rc != 0:
        raise ValueError("symmetric oracle rejected the cycle list (rc=%d)" % rc)
    return out
