"""Pins of the symmetric band -> tridiagonal oracle (page "A two-stage
reduction on an Apple M5 Pro", section 6, the symmetric-band kernels) to
facts other than itself:
  * an independent dense Householder tridiagonalization (written here) whose
    reflectors also leave index 0 alone: by the implicit-Q theorem T is then
    unique up to the signs of e, so d and |e| agree elementwise;
  * eigenvalues of T equal numpy's eigenvalues of the dense matrix;
  * Frobenius-norm invariance, exact zeros off the tridiagonal;
  * TW-invariance of d and |e|; BW = 0 and 1 are copies; zero bands and
    zero rows; n <= 3 and full bands;
  * schedules: the footprints of the cycles (every entry a cycle reads or
    writes) show that sweep R may run cycle k once sweep R-1 has completed
    min(k + L, all) cycles, L = 2 when b' >= 2 and 3 when b' = 1, with the
    final count published after the predecessor's; split into half-cycles
    (pivot row and row segments; block and column segments) the lag is
    d = 2, 3, 4 halves for b' >= 3, 2, 1; one unit less is never enough; and
    an order that runs concurrent cycles in reverse reproduces the
    sequential result to the bit.
Planted mistakes in a copy of the oracle each fail this battery
(test_planted_mistake_is_caught).
"""
import os
import shutil
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import bb_inputs
import oracle
from refs import pass_list

SHAPES = [(30, 6, 2), (40, 8, 3), (33, 5, 4), (40, 8, 7), (25, 4, 1), (64, 16, 8), (100, 9, 4), (50, 12, 1),
          (45, 20, 7), (17, 16, 15)]


def dense_sym(band, bw):
    n = band.shape[0]
    A = np.zeros((n, n))
    for i in range(n):
        for o in range(bw + 1):
            if i + o < n:
                A[i, i + o] = A[i + o, i] = band[i, o]
    return A


def dense_householder_tridiag(A):
    """Textbook tridiagonalization: column k's entries below k+1 annihilated
    by a reflector on rows/columns k+1..n-1 (never index 0)."""
    A = A.copy()
    n = A.shape[0]
    for k in range(n - 2):
        x = A[k + 1:, k].copy()
        nrm = np.linalg.norm(x)
        if nrm == 0 or np.linalg.norm(x[1:]) == 0:
            continue
        u = x.copy()
        u[0] += np.copysign(nrm, x[0])
        u /= np.linalg.norm(u)
        A[k + 1:, :] -= 2.0 * np.outer(u, u @ A[k + 1:, :])
        A[:, k + 1:] -= 2.0 * np.outer(A[:, k + 1:] @ u, u)
    return np.diag(A).copy(), np.diag(A, 1).copy()


@pytest.mark.parametrize("n,bw,tw", SHAPES)
def test_matches_dense_householder_and_eigenvalues(n, bw, tw):
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=n + bw)
    A = dense_sym(band, bw)
    d, e = oracle.sym_reduce(band, bw, tw)
    dd, de = dense_householder_tridiag(A)
    scale = np.linalg.norm(A)
    assert np.max(np.abs(d - dd)) <= 1e-12 * scale
    assert np.max(np.abs(np.abs(e) - np.abs(de))) <= 1e-12 * scale
    ev = np.linalg.eigvalsh(A)
    et = np.linalg.eigvalsh(np.diag(d) + np.diag(e, 1) + np.diag(e, -1))
    assert np.max(np.abs(ev - et)) <= 1e-12 * scale


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("n,bw,tw", SHAPES[:6])
def test_exact_zeros_and_norm(n, bw, tw, dt):
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=3)
    d, e, W = oracle.sym_reduce(band, bw, tw, return_band=True)
    assert np.all(W[:, 2:] == 0)
    np.testing.assert_array_equal(W[:, 0], d)
    np.testing.assert_array_equal(W[:-1, 1], e)
    A = dense_sym(band.astype(np.float64), bw)
    fro = float(np.sum(d.astype(np.float64) ** 2) + 2 * np.sum(e.astype(np.float64) ** 2))
    eps = np.finfo(bb_inputs.np_dtype(dt)).eps
    assert abs(fro - np.sum(A * A)) <= 50 * n * eps * np.sum(A * A)


def test_tile_width_invariance():
    n, bw = 80, 12
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=11)
    d0, e0 = oracle.sym_reduce(band, bw, 1)
    for tw in (2, 3, 5, 11, 40):
        d, e = oracle.sym_reduce(band, bw, tw)
        assert np.max(np.abs(d - d0)) <= 1e-12 * np.max(np.abs(d0))
        assert np.max(np.abs(np.abs(e) - np.abs(e0))) <= 1e-12 * np.max(np.abs(d0))


def test_special_cases():
    band = bb_inputs.make_band(20, 0, "f64", "normal", seed=1)
    d, e = oracle.sym_reduce(band, 0, 4)
    np.testing.assert_array_equal(d, band[:, 0])
    assert np.all(e == 0)
    band = bb_inputs.make_band(20, 1, "f64", "normal", seed=2)
    d, e = oracle.sym_reduce(band, 1, 4)
    np.testing.assert_array_equal(d, band[:, 0])
    np.testing.assert_array_equal(e, band[:-1, 1])
    z = np.zeros((30, 7))
    d, e = oracle.sym_reduce(z, 6, 3)
    assert np.all(d == 0) and np.all(e == 0)
    for n in (1, 2, 3):
        band = bb_inputs.make_band(n, 4, "f64", "normal", seed=n)
        d, e = oracle.sym_reduce(band, 4, 2)
        A = dense_sym(band, 4)
        et = np.linalg.eigvalsh(np.diag(d) + np.diag(e, 1) + np.diag(e, -1))
        assert np.allclose(et, np.linalg.eigvalsh(A), atol=1e-14)
    # zero rows (and their columns) take identity reflectors
    band = bb_inputs.make_band(60, 8, "f64", "normal", seed=4)
    A0 = dense_sym(band, 8)
    for i in (5, 17, 30):
        band[i, :] = 0
        if i >= 1:
            for o in range(1, 9):
                if i - o >= 0:
                    band[i - o, o] = 0
    A = dense_sym(band, 8)
    assert np.all(A[[5, 17, 30], :] == 0) and not np.array_equal(A, A0)
    d, e = oracle.sym_reduce(band, 8, 3)
    et = np.linalg.eigvalsh(np.diag(d) + np.diag(e, 1) + np.diag(e, -1))
    assert np.allclose(et, np.linalg.eigvalsh(A), atol=1e-12)


# ---- schedules ----------------------------------------------------------------

def cycles_of(n, b, t, R):
    last = n - 2 - R - (b - t)
    return 0 if last < 0 else last // b + 1


def footprint(n, b, t, R, k):
    """Every upper-triangle entry cycle (R, k) reads or writes."""
    c = R + (b - t) + k * b
    ch = min(c + t, n - 1)
    p = R if k == 0 else c - b
    out = set()
    for i in range(p, c):
        out.update((i, j) for j in range(c, ch + 1))
    for i in range(c, ch + 1):
        out.update((i, j) for j in range(i, min(ch + b, n - 1) + 1))
    return out


def done_when_starting(K, L, R2, k2, R1):
    """Cycles of sweep R1 < R2 certainly complete when (R2, k2) starts."""
    need = min(k2 + L, K[R2 - 1])
    R = R2 - 1
    while R > R1:
        if need == K[R]:
            return K[R1]          # R complete: every earlier sweep complete
        if need == 0:
            return 0
        need = min(need - 1 + L, K[R - 1])
        R -= 1
    return need


def conflicts_unordered(n, b, t, L):
    ns = max(n - (b - t) - 1, 0)
    K = [cycles_of(n, b, t, R) for R in range(ns)]
    fp = {(R, k): footprint(n, b, t, R, k) for R in range(ns) for k in range(K[R])}
    bad = []
    for (R2, k2), f2 in fp.items():
        for R1 in range(max(0, R2 - 6), R2):
            done = done_when_starting(K, L, R2, k2, R1)
            for k1 in range(done, K[R1]):
                if fp[(R1, k1)] & f2:
                    bad.append(((R1, k1), (R2, k2)))
    return bad


@pytest.mark.parametrize("n,b,t", [(40, 6, 2), (40, 6, 4), (45, 8, 7), (30, 5, 3), (36, 4, 1), (33, 3, 2),
                                   (40, 2, 1), (50, 9, 4), (27, 7, 6)])
def test_wait_rule_orders_every_conflict(n, b, t):
    L = 2 if b - t >= 2 else 3
    assert conflicts_unordered(n, b, t, L) == []
    assert conflicts_unordered(n, b, t, L - 1) != []   # one cycle less is not enough


def half_footprint(n, b, t, R, q):
    """Entries half q of sweep R reads or writes: half 2k is the pivot row
    and the row segments above the block, half 2k+1 the block and the
    column segments to its right (both of cycle k)."""
    k, h = divmod(q, 2)
    c = R + (b - t) + k * b
    ch = min(c + t, n - 1)
    p = R if k == 0 else c - b
    out = set()
    if h == 0:
        for i in range(p, c):
            out.update((i, j) for j in range(c, ch + 1))
    else:
        for i in range(c, ch + 1):
            out.update((i, j) for j in range(i, min(ch + b, n - 1) + 1))
    return out


def half_conflicts_unordered(n, b, t, d):
    ns = max(n - (b - t) - 1, 0)
    K2 = [2 * cycles_of(n, b, t, R) for R in range(ns)]
    fp = {(R, q): half_footprint(n, b, t, R, q) for R in range(ns) for q in range(K2[R])}
    bad = []
    for (R2, q2), f2 in fp.items():
        for R1 in range(max(0, R2 - 8), R2):
            done = done_when_starting(K2, d, R2, q2, R1)
            for q1 in range(done, K2[R1]):
                if fp[(R1, q1)] & f2:
                    bad.append(((R1, q1), (R2, q2)))
    return bad


@pytest.mark.parametrize("n,b,t", [(40, 6, 2), (40, 6, 4), (45, 8, 7), (30, 5, 3), (36, 4, 1), (33, 3, 2),
                                   (40, 2, 1), (60, 16, 13), (60, 16, 14), (60, 16, 15)])
def test_half_cycle_rule_orders_every_conflict(n, b, t):
    # at half-cycle granularity the lag is d = 2 / 3 / 4 half-cycles for
    # b' >= 3 / 2 / 1, the rule of the general band; one less is not enough
    bp = b - t
    d = 2 if bp >= 3 else (3 if bp == 2 else 4)
    assert half_conflicts_unordered(n, b, t, d) == []
    assert half_conflicts_unordered(n, b, t, d - 1) != []


@pytest.mark.parametrize("n,bw,tw", [(40, 8, 3), (33, 6, 5), (30, 5, 1)])
def test_concurrent_cycles_commute_to_the_bit(n, bw, tw):
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=7)
    ref = oracle.sym_reduce(band, bw, tw, return_band=True)[2]
    order = []
    for ps, (b, t) in enumerate(pass_list(bw, tw)):
        s = 2 if b - t >= 2 else 3
        ns = max(n - (b - t) - 1, 0)
        K = [cycles_of(n, b, t, R) for R in range(ns)]
        for step in range(max(k + s * R for R in range(ns) for k in range(K[R])) + 1 if ns else 0):
            for R in reversed(range(ns)):
                k = step - s * R
                if 0 <= k < K[R]:
                    order.append((ps, R, k))
    np.testing.assert_array_equal(oracle.sym_run_cycles(band, bw, tw, order), ref)


# ---- planted mistakes ---------------------------------------------------------------

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BODY = "bb_oracle_sym_body.h"
MUTANTS = {
    "left_range_short": ("for (int64_t j = ch + 1; j <= smin64(ch + b, n - 1); ++j)",
                         "for (int64_t j = ch + 1; j <= smin64(ch + b - 1, n - 1); ++j)"),
    "right_rows_start": ("for (int64_t i = p + 1; i < c; ++i)", "for (int64_t i = p + 2; i < c; ++i)"),
    "chase_column": ("const int64_t p = (k == 0) ? R : c - b;", "const int64_t p = (k == 0) ? R : c - b + 1;"),
    "rank2_half": ("const REAL alpha = -(((REAL)0.5 * tau) * dot);", "const REAL alpha = -(tau * dot);"),
    "rank2_one_side": ("*e = SFMA(-v[i], z[j], SFMA(-z[i], v[j], *e));", "*e = SFMA(-z[i], v[j], *e);"),
    "tau_sign": ("*tau = (bt - alpha) / bt;", "*tau = (alpha - bt) / bt;"),
    "unscaled_vector": ("v[j] = x[j] * inv;", "v[j] = x[j];"),
}

BATTERY = textwrap.dedent(r'''
    import ctypes, sys
    import numpy as np
    sys.path.insert(0, sys.argv[2])
    import bb_inputs
    L = ctypes.CDLL(sys.argv[1])
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    L.bb_oracle_sym_reduce_f64.argtypes = [vp, i64, i64, i32, i32, vp, vp, vp]
    for (n, bw, tw) in [(30, 6, 2), (40, 8, 7), (25, 4, 1), (64, 16, 8)]:
        band = bb_inputs.make_band(n, bw, "f64", "normal", seed=n)
        A = np.zeros((n, n))
        for i in range(n):
            for o in range(bw + 1):
                if i + o < n:
                    A[i, i + o] = A[i + o, i] = band[i, o]
        d = np.zeros(n); e = np.zeros(n - 1)
        assert L.bb_oracle_sym_reduce_f64(band.ctypes.data, band.shape[1], n, bw, tw, d.ctypes.data,
                                          e.ctypes.data, None) == 0
        et = np.linalg.eigvalsh(np.diag(d) + np.diag(e, 1) + np.diag(e, -1))
        assert np.max(np.abs(et - np.linalg.eigvalsh(A))) <= 1e-12 * np.linalg.norm(A)
''')


def _run_battery(tmp_path, subst=None):
    src = tmp_path / "src"
    src.mkdir()
    for f in ("bb_oracle_sym.c", BODY):
        shutil.copy(os.path.join(ROOT, "oracle", f), src / f)
    if subst:
        text = (src / BODY).read_text()
        assert text.count(subst[0]) == 1, subst[0]
        (src / BODY).write_text(text.replace(subst[0], subst[1]))
    so = tmp_path / "m.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-mfma", "-fno-math-errno",
                    "-o", str(so), str(src / "bb_oracle_sym.c"), "-lm"], check=True)
    script = tmp_path / "battery.py"
    script.write_text(BATTERY)
    return subprocess.run([sys.executable, str(script), str(so), ROOT], capture_output=True,
                          timeout=300).returncode


def test_real_oracle_passes_mutant_battery(tmp_path):
    assert _run_battery(tmp_path) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    assert _run_battery(tmp_path, MUTANTS[name]) != 0, name
