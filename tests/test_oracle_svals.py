"""Pins of the bisection oracle (bidiagonal -> singular values, page "A
two-stage reduction on an Apple M5 Pro", section 7) to facts other than
itself:
  * closed form: d = e = 1 gives sigma_k = 2 cos(k pi / (2n + 1)) (the
    Golub-Kahan tridiagonal is then the all-ones Toeplitz tridiagonal);
  * a diagonal B has sigma = sorted |d|; a 2 x 2 B has sigma_1 sigma_2 = |ab|
    and sigma_1^2 + sigma_2^2 = ||B||_F^2;
  * LAPACK's bisection (dstebz through SciPy) on the same tridiagonal agrees
    to an ulp of the norm, and the dense SVD to its own backward error;
  * the fp32 oracle is within a few fp32 ulps of the norm of the fp64 truth
    (the page's accuracy claim for its float32 bisection);
  * the Sturm count equals the number of eigenvalues <= x of the dense
    tridiagonal, and the interval holds the whole spectrum;
  * signs of d and e change nothing (bitwise); singular B gives a zero;
  * n = 0, 1 and index ranges.
Planted mistakes (a swapped off-diagonal order, an index off by one, a
missing square, a wrong first pivot, a radius without the neighbour, too few
halvings) each fail this battery; see test_planted_mistake_is_caught.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import numpy as np
import pytest
import scipy.linalg as sl

import oracle

EPS = {np.float64: np.finfo(np.float64).eps, np.float32: np.finfo(np.float32).eps}


def gk_offdiag(d, e):
    n = d.size
    b = np.empty(2 * n - 1, dtype=np.float64)
    b[0::2] = d
    b[1::2] = e
    return b


def random_bidiag(n, seed, dtype=np.float64):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(n).astype(dtype), rng.standard_normal(max(n - 1, 0)).astype(dtype)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
@pytest.mark.parametrize("n", [1, 2, 3, 8, 51, 300])
def test_closed_form_all_ones(n, dtype):
    s = oracle.svals(np.ones(n, dtype), np.ones(n - 1, dtype))
    ref = 2 * np.cos(np.arange(1, n + 1) * np.pi / (2 * n + 1))
    assert s.dtype == dtype
    assert np.max(np.abs(s - ref)) <= 3 * EPS[dtype] * 2


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_diagonal_and_two_by_two(dtype):
    rng = np.random.default_rng(5)
    d = rng.standard_normal(40).astype(dtype)
    s = oracle.svals(d, np.zeros(39, dtype))
    ref = np.sort(np.abs(d.astype(np.float64)))[::-1]
    assert np.max(np.abs(s - ref)) <= 2 * EPS[dtype] * ref[0]
    a, b, c = dtype(1.5), dtype(-0.25), dtype(2.0)
    s1, s2 = oracle.svals(np.array([a, b]), np.array([c])).astype(np.float64)
    assert abs(s1 * s2 - abs(float(a) * float(b))) <= 8 * EPS[dtype] * s1 * s1
    assert abs(s1 * s1 + s2 * s2 - (a * a + b * b + c * c)) <= 8 * EPS[dtype] * s1 * s1


@pytest.mark.parametrize("n", [5, 64, 257, 1000])
def test_matches_lapack_bisection_and_dense_svd(n):
    d, e = random_bidiag(n, n)
    s = oracle.svals(d, e)
    stebz = sl.eigvalsh_tridiagonal(np.zeros(2 * n), gk_offdiag(d, e), lapack_driver="stebz")[::-1][:n]
    svd = np.linalg.svd(np.diag(d) + np.diag(e, 1), compute_uv=False)
    eps = EPS[np.float64]
    assert np.max(np.abs(s - stebz)) <= 2 * eps * svd[0]
    assert np.max(np.abs(s - svd)) <= n * eps * svd[0]
    assert np.all(np.diff(s) <= 0)


def test_fp32_within_a_few_ulps_of_the_norm():
    n = 1500
    d, e = random_bidiag(n, 9)
    d32, e32 = d.astype(np.float32), e.astype(np.float32)
    truth = sl.eigvalsh_tridiagonal(np.zeros(2 * n), gk_offdiag(d32.astype(np.float64), e32.astype(np.float64)),
                                    lapack_driver="stebz")[::-1][:n]
    s = oracle.svals(d32, e32).astype(np.float64)
    assert np.max(np.abs(s - truth)) <= 2 * EPS[np.float32] * truth[0]


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_sturm_count_and_interval(dtype):
    n = 60
    d, e = random_bidiag(n, 2, dtype)
    lo, hi, pm = oracle.gk_interval(d, e)
    ev = np.linalg.eigvalsh(np.diag(gk_offdiag(d, e), 1) + np.diag(gk_offdiag(d, e), -1))
    assert lo == -hi and hi > ev[-1] and lo < ev[0]
    assert pm == np.finfo(dtype).tiny * max(1.0, float(np.max(gk_offdiag(d, e).astype(dtype) ** 2)))
    assert oracle.gk_count(d, e, lo, pm) == 0 and oracle.gk_count(d, e, hi, pm) == 2 * n
    rng = np.random.default_rng(3)
    gap = 1e-3 * ev[-1]
    for x in rng.uniform(lo, hi, 200):
        if np.min(np.abs(ev - x)) < gap:
            continue
        assert oracle.gk_count(d, e, x, pm) == int(np.sum(ev <= x))


def test_signs_change_nothing():
    d, e = random_bidiag(200, 4)
    rng = np.random.default_rng(8)
    sd, se = rng.choice([-1.0, 1.0], d.size), rng.choice([-1.0, 1.0], e.size)
    assert np.array_equal(oracle.svals(d, e), oracle.svals(d * sd, e * se))


def test_singular_and_zero_bidiagonals():
    d, e = random_bidiag(30, 6)
    d[11] = 0.0
    s = oracle.svals(d, e)
    assert s[-1] >= 0 and s[-1] <= 4 * EPS[np.float64] * s[0]
    z = oracle.svals(np.zeros(7), np.zeros(6))
    _, _, pm = oracle.gk_interval(np.zeros(7), np.zeros(6))
    assert np.all(z >= 0) and np.all(z <= 2 * pm)


def test_sizes_and_ranges():
    assert oracle.svals(np.zeros(0), np.zeros(0)).size == 0
    assert oracle.svals(np.array([-3.0]), np.zeros(0))[0] == 3.0
    d, e = random_bidiag(50, 1)
    full = oracle.svals(d, e)
    assert np.array_equal(oracle.svals(d, e, 10, 23), full[10:23])
    assert oracle.svals(d, e, 7, 7).size == 0
    with pytest.raises(ValueError):
        oracle.svals(d, e, 3, 51)
    with pytest.raises(ValueError):
        oracle.svals(d, e[:-1])


# ---------------------------------------------------------------------------
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BODY = "bb_oracle_svals_body.h"
MUTANTS = {
    "offdiag_order_swapped": ("return (j % 2 == 1) ? d[(j - 1) / 2] : e[j / 2 - 1];",
                              "return (j % 2 == 0) ? d[j / 2 - 1] : (j / 2 < n - 1 ? e[j / 2] : d[n - 1]);"),
    "index_off_by_one": ("const int64_t j = 2 * n - i;", "const int64_t j = 2 * n - i - 1;"),
    "missing_square": ("q = -((b * b) / q) - x;", "q = -(fabs(b) / q) - x;"),
    "first_pivot_sign": ("REAL q = -x;", "REAL q = x;"),
    "radius_without_neighbour": ("if (left + right > r) r = left + right;", "if (right > r) r = right;"),
    "too_few_halvings": ("h < REAL_HALVINGS;", "h < REAL_HALVINGS - 12;"),
}

BATTERY = textwrap.dedent(r'''
    import ctypes, sys
    import numpy as np
    import scipy.linalg as sl
    L = ctypes.CDLL(sys.argv[1])
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.bb_oracle_svals_f64.argtypes = [vp, vp, i64, i64, i64, vp]
    def sv(d, e):
        out = np.zeros(d.size)
        assert L.bb_oracle_svals_f64(d.ctypes.data, e.ctypes.data, d.size, 0, d.size, out.ctypes.data) == 0
        return out
    eps = np.finfo(float).eps
    for n in (3, 40):
        s = sv(np.ones(n), np.ones(n - 1))
        assert np.max(np.abs(s - 2 * np.cos(np.arange(1, n + 1) * np.pi / (2 * n + 1)))) <= 6 * eps
    rng = np.random.default_rng(0)
    for n in (2, 17, 120):
        d, e = rng.standard_normal(n), rng.standard_normal(n - 1)
        b = np.empty(2 * n - 1); b[0::2] = d; b[1::2] = e
        ref = sl.eigvalsh_tridiagonal(np.zeros(2 * n), b, lapack_driver="stebz")[::-1][:n]
        assert np.max(np.abs(sv(d, e) - ref)) <= 2 * eps * ref[0]
''')


def _run_battery(tmp_path, subst=None):
    src = tmp_path / "src"
    src.mkdir()
    for f in ("bb_oracle_svals.c", BODY):
        shutil.copy(os.path.join(ROOT, "oracle", f), src / f)
    if subst:
        text = (src / BODY).read_text()
        assert text.count(subst[0]) == 1, subst[0]
        (src / BODY).write_text(text.replace(subst[0], subst[1]))
    so = tmp_path / "m.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-mfma",
                    "-fno-math-errno", "-o", str(so), str(src / "bb_oracle_svals.c"), "-lm"], check=True)
    script = tmp_path / "battery.py"
    script.write_text(BATTERY)
    return subprocess.run([sys.executable, str(script), str(so)], capture_output=True, timeout=300).returncode


def test_real_oracle_passes_mutant_battery(tmp_path):
    assert _run_battery(tmp_path) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    assert _run_battery(tmp_path, MUTANTS[name]) != 0, name
