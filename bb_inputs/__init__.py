"""Seeded synthetic upper-band inputs shared by the oracle tests and the HIP path.

This module holds no arithmetic of the reduction itself: it only draws band
entries and names the workloads.  A band is returned in the row-offset layout
both sides consume: an (n, bw+1) array whose row i holds A(i, i..i+bw); the
entries with i+o >= n (outside the matrix) are zero.

Recipe (every workload is synthetic; the pages name no public dataset):
  * numpy.random.default_rng(seed), PCG64, seed 0 unless stated;
  * draw an (n, bw+1) float64 array in row-major order from the workload's
    distribution, zero the entries past the matrix edge;
  * 'graded':  multiply A(i,j) by 10**(-6 j / n), j = i+o the absolute column,
    in float64, giving singular values graded over six decades;
  * 'uniform_zero_rows': U(-1,1) entries, then round(0.01 n) distinct rows
    drawn with rng.choice(n, ., replace=False) after the band draw get all
    their band entries set to +0.0 (exercises zero reflectors);
  * cast once to the workload's dtype.  Both the oracle and the GPU consume
    the same cast array.

Bidiagonals for the singular-value step (make_bidiag): d (n) then e (n-1)
drawn from one default_rng(seed) stream, N(0,1) ('normal'), the same times
10**(-6 i / n) for entry i ('graded'), or all ones ('ones'); cast once.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    n: int
    bw: int
    tw: int
    dtype: str  # 'f32' or 'f64'
    dist: str  # 'normal', 'graded', 'uniform_zero_rows'
    seed: int = 0


# The five workloads the method is measured on, named by what they are.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("n512-bw16-tw8-f64-normal", 512, 16, 8, "f64", "normal"),
        Workload("n4096-bw32-tw16-f32-normal", 4096, 32, 16, "f32", "normal"),
        Workload("n16384-bw64-tw16-f32-normal", 16384, 64, 16, "f32", "normal"),
        Workload("n32768-bw128-tw32-f64-graded", 32768, 128, 32, "f64", "graded"),
        Workload("n65536-bw256-tw32-f32-zerorows", 65536, 256, 32, "f32", "uniform_zero_rows"),
    )
}

HEADLINE = "n16384-bw64-tw16-f32-normal"


def np_dtype(name: str):
    return {"f32": np.float32, "f64": np.float64}[name]


def make_band(n: int, bw: int, dtype: str = "f64", dist: str = "normal", seed: int = 0) -> np.ndarray:
    """Seeded (n, bw+1) upper band in row-offset layout, cast to dtype."""
    rng = np.random.default_rng(seed)
    shape = (n, bw + 1)
    if dist in ("normal", "graded"):
        a = rng.standard_normal(shape)
    elif dist in ("uniform", "uniform_zero_rows"):
        a = rng.uniform(-1.0, 1.0, shape)
    else:
        raise ValueError("unknown distribution %r" % dist)
    i = np.arange(n)[:, None]
    o = np.arange(bw + 1)[None, :]
    a[i + o >= n] = 0.0
    if dist == "graded":
        a *= 10.0 ** (-6.0 * (i + o) / n)
        a[i + o >= n] = 0.0
    if dist == "uniform_zero_rows":
        nz = int(round(0.01 * n))
        rows = rng.choice(n, nz, replace=False)
        a[rows, :] = 0.0
    return np.ascontiguousarray(a.astype(np_dtype(dtype)))


def make_bidiag(n: int, dtype: str = "f64", dist: str = "normal", seed: int = 0):
    """Seeded upper bidiagonal (d, e) for the singular-value step."""
    rng = np.random.default_rng(seed)
    if dist == "ones":
        d, e = np.ones(n), np.ones(max(n - 1, 0))
    elif dist in ("normal", "graded"):
        d, e = rng.standard_normal(n), rng.standard_normal(max(n - 1, 0))
        if dist == "graded":
            d *= 10.0 ** (-6.0 * np.arange(n) / max(n, 1))
            e *= 10.0 ** (-6.0 * np.arange(e.size) / max(n, 1))
    else:
        raise ValueError("unknown distribution %r" % dist)
    return d.astype(np_dtype(dtype)), e.astype(np_dtype(dtype))


def make_workload(w: Workload | str) -> np.ndarray:
    if isinstance(w, str):
        w = WORKLOADS[w]
    return make_band(w.n, w.bw, w.dtype, w.dist, w.seed)


def zero_rows(w: Workload | str) -> np.ndarray:
    """Indices of the rows zeroed by the 'uniform_zero_rows' recipe."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    rng.uniform(-1.0, 1.0, (w.n, w.bw + 1))
    return np.sort(rng.choice(w.n, int(round(0.01 * w.n)), replace=False))
