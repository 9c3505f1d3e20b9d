"""Independent reference computations used to pin the oracle (test-only).

None of this shares code with the oracle or the HIP library:
  * dense_golub_kahan: textbook dense Householder bidiagonalization of the full
    matrix (left reflector on column k, then right reflector on row k).  Its
    right transform fixes e_1, as the band method's does (right reflectors
    only touch columns >= 1), so |d| and |e| must agree with the band method
    whenever the bidiagonal is unreduced (Golub-Kahan-Lanczos uniqueness).
  * jacobi_singular_values: brute-force one-sided Jacobi SVD.
  * bidiag_singular_values: singular values of an upper bidiagonal through the
    2n x 2n Golub-Kahan tridiagonal (zero diagonal, off-diagonal d0,e0,d1,...),
    whose non-negative eigenvalues are the singular values.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


def dense_from_band(band: np.ndarray, bw: int) -> np.ndarray:
    n = band.shape[0]
    A = np.zeros((n, n), dtype=np.float64)
    for i in range(n):
        for o in range(bw + 1):
            if i + o < n:
                A[i, i + o] = band[i, o]
    return A


def _house_vec(x):
    nx = np.linalg.norm(x)
    if x.size < 2 or np.linalg.norm(x[1:]) == 0.0:
        return None
    v = x.astype(np.float64).copy()
    v[0] += np.copysign(nx, x[0])
    return v / np.linalg.norm(v)


def dense_golub_kahan(A: np.ndarray):
    A = np.array(A, dtype=np.float64)
    n = A.shape[0]
    for k in range(n):
        v = _house_vec(A[k:, k])
        if v is not None:
            A[k:, :] -= 2.0 * np.outer(v, v @ A[k:, :])
        if k + 2 <= n - 1:
            v = _house_vec(A[k, k + 1:])
            if v is not None:
                A[:, k + 1:] -= 2.0 * np.outer(A[:, k + 1:] @ v, v)
    return np.diag(A).copy(), np.diag(A, 1).copy()


def jacobi_singular_values(A: np.ndarray, sweeps: int = 60) -> np.ndarray:
    """One-sided Jacobi: rotate column pairs until mutually orthogonal."""
    U = np.array(A, dtype=np.float64)
    n = U.shape[1]
    for _ in range(sweeps):
        off = 0.0
        for p in range(n - 1):
            for q in range(p + 1, n):
                alpha = U[:, p] @ U[:, p]
                beta = U[:, q] @ U[:, q]
                gamma = U[:, p] @ U[:, q]
                if gamma == 0.0:
                    continue
                off = max(off, abs(gamma) / np.sqrt(alpha * beta))
                zeta = (beta - alpha) / (2.0 * gamma)
                t = np.copysign(1.0, zeta) / (abs(zeta) + np.sqrt(1.0 + zeta * zeta))
                c = 1.0 / np.sqrt(1.0 + t * t)
                s = c * t
                up = U[:, p].copy()
                U[:, p] = c * up - s * U[:, q]
                U[:, q] = s * up + c * U[:, q]
        if off < 1e-15:
            break
    return np.sort(np.linalg.norm(U, axis=0))[::-1]


def bidiag_singular_values(d: np.ndarray, e: np.ndarray) -> np.ndarray:
    d = np.asarray(d, dtype=np.float64)
    e = np.asarray(e, dtype=np.float64)
    n = d.size
    if n == 1:
        return np.abs(d)
    off = np.zeros(2 * n - 1)
    off[0::2] = d
    off[1::2] = e
    ev = scipy.linalg.eigvalsh_tridiagonal(np.zeros(2 * n), off, lapack_driver="sterf")
    # eigenvalues come in +-sigma pairs: keep the n largest (non-negative)
    return np.sort(ev)[::-1][:n].copy()


def pass_list(bw: int, tw: int):
    """(b, t) per pass: t = min(TW, b-1), b -> b - t until b = 1."""
    out = []
    b = bw
    while b > 1:
        t = min(tw, b - 1)
        out.append((b, t))
        b -= t
    return out


def cycles_of_sweep(n: int, b: int, t: int, R: int) -> int:
    bp = b - t
    k = 0
    while R + bp + k * b <= n - 2:
        k += 1
    return k


def sequential_order(n: int, bw: int, tw: int):
    order = []
    for p, (b, t) in enumerate(pass_list(bw, tw)):
        bp = b - t
        for R in range(0, max(n - bp - 1, 0)):
            for k in range(cycles_of_sweep(n, b, t, R)):
                order.append((p, R, k))
    return order


def staggered_order(n: int, bw: int, tw: int, stagger: int, reverse_within_step: bool = True):
    """Order of a one-launch-per-step schedule: step L runs every (R, k = L - stagger*R).

    Within a step the cycles are emitted from the largest R down (or up) so
    that a dependence violated inside a step shows up as a result change."""
    order = []
    for p, (b, t) in enumerate(pass_list(bw, tw)):
        bp = b - t
        nsw = max(n - bp - 1, 0)
        K = [cycles_of_sweep(n, b, t, R) for R in range(nsw)]
        steps = max((stagger * R + K[R] for R in range(nsw)), default=0)
        for L in range(steps):
            rs = range(nsw - 1, -1, -1) if reverse_within_step else range(nsw)
            for R in rs:
                k = L - stagger * R
                if 0 <= k < K[R]:
                    order.append((p, R, k))
    return order


def cycle_window(n: int, b: int, t: int, R: int, k: int):
    """Set of (i, j) entries one cycle reads or writes."""
    bp = b - t
    c = R + bp + k * b
    ch = min(c + t, n - 1)
    r = R if k == 0 else c - b
    cells = set()
    for j in range(c, ch + 1):
        cells.add((r, j))
    for i in range(r + 1, ch + 1):
        for j in range(c, ch + 1):
            cells.add((i, j))
    for i in range(c, ch + 1):
        for j in range(c, min(c + t + b, n - 1) + 1):
            cells.add((i, j))
    return cells
