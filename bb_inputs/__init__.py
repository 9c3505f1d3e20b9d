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

Bands with known singular values (known_spectrum_band), for the accuracy
study of the reduced-precision reduction: A = U diag(sigma) V^T with U, V
the Q factors of seeded Gaussian matrices (signs fixed by R's diagonal),
sigma in [0, 1] from one of three spectra ('arithmetic': 1 - i/n;
'logarithmic': 10**(-6 i/(n-1)); 'quarter_circle': n draws from the density
(4/pi) sqrt(1 - s^2) on [0, 1], by rejection, sorted), reduced to an upper
band of bandwidth bw in fp64 by the classical block Householder first stage
(QR of each column panel, then LQ of the row panel to its right), entries
beyond the band dropped (they are rounding noise).

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
    return {"f16": np.float16, "f32": np.float32, "f64": np.float64}[name]


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


SPECTRA = ("arithmetic", "logarithmic", "quarter_circle")


def _orthogonal(n: int, rng) -> np.ndarray:
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))[None, :]


def known_spectrum(n: int, spectrum: str, rng) -> np.ndarray:
    i = np.arange(n, dtype=np.float64)
    if spectrum == "arithmetic":
        return 1.0 - i / n
    if spectrum == "logarithmic":
        return 10.0 ** (-6.0 * i / max(n - 1, 1))
    if spectrum == "quarter_circle":
        out = []
        while len(out) < n:
            s, u = rng.uniform(0.0, 1.0, 2 * n), rng.uniform(0.0, 1.0, 2 * n)
            out.extend(s[u <= np.sqrt(1.0 - s * s)].tolist())
        return np.sort(np.asarray(out[:n]))[::-1].copy()
    raise ValueError("unknown spectrum %r" % spectrum)


def dense_to_band(A: np.ndarray, bw: int) -> np.ndarray:
    """Upper band (n, bw+1), row i = A'(i, i..i+bw), of A' = Q^T A P from
    block Householder panels of width bw (fp64)."""
    A = np.array(A, dtype=np.float64)
    n = A.shape[0]
    for j in range(0, n, bw):
        q, _ = np.linalg.qr(A[j:, j:j + bw], mode="complete")
        A[j:, j:] = q.T @ A[j:, j:]
        if j + bw < n:
            q2, _ = np.linalg.qr(A[j:j + bw, j + bw:].T, mode="complete")
            A[:, j + bw:] = A[:, j + bw:] @ q2
    band = np.zeros((n, bw + 1))
    for o in range(bw + 1):
        band[:n - o, o] = np.diagonal(A, o)
    return band


def known_spectrum_band(n: int, bw: int, spectrum: str, seed: int = 0):
    """(band in fp64, sigma descending) with the band's singular values sigma."""
    rng = np.random.default_rng(seed)
    sigma = known_spectrum(n, spectrum, rng)
    U, V = _orthogonal(n, rng), _orthogonal(n, rng)
    A = (U * sigma[None, :]) @ V.T
    return dense_to_band(A, bw), sigma


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
