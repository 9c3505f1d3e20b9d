"""Pins of the CPU oracle to facts fixed by mathematics and by the pages.

The oracle is checked here against things other than itself:
  * an independent dense Golub-Kahan bidiagonalization (uniqueness of B up to
    signs when the right transform fixes e_1): |d|, |e| elementwise;
  * brute-force one-sided Jacobi singular values and LAPACK's SVD of the
    dense matrix;
  * orthogonal invariance of the Frobenius norm;
  * exact zeros everywhere off the diagonal and superdiagonal;
  * invariance of |d|, |e| under the tile width TW (every TW reaches the same
    unique bidiagonal);
  * exact scaling by powers of two;
  * special cases: BW = 0, BW = 1, all-zero bands, zero rows, n = 1, 2,
    n <= BW + 1, TW >= BW;
  * the pass list of the 512 x 512 workload, 16 -> 8 -> 1, as stated with it;
  * schedules: the three-cycle separation keeps concurrent cycles disjoint
    (page "Accelerating Bidiagonalization ... on GPUs", three-cycle
    separation passage), two cycles suffice only when the target band is
    wider than bidiagonal, and every valid schedule reproduces the
    sequential result to the bit.
"""
import numpy as np
import pytest

import bb_inputs
import oracle
from refs import (bidiag_singular_values, cycle_window, cycles_of_sweep, dense_from_band,
                  dense_golub_kahan, jacobi_singular_values, pass_list, sequential_order,
                  staggered_order)

SHAPES = [(40, 6, 2), (64, 16, 8), (100, 9, 4), (30, 5, 10), (50, 12, 1), (7, 3, 1),
          (96, 12, 5), (33, 32, 16), (45, 20, 7)]


def off_bidiag_max(work, T):
    n, ld = work.shape
    m = 0.0
    for o in range(ld):
        if o - T in (0, 1):
            continue
        m = max(m, float(np.max(np.abs(work[:, o]))))
    return m


@pytest.mark.parametrize("n,bw,tw", SHAPES)
def test_matches_dense_golub_kahan(n, bw, tw):
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=3)
    A = dense_from_band(band, bw)
    d, e = oracle.reduce(band, bw, tw)
    dg, eg = dense_golub_kahan(A)
    fro = np.linalg.norm(A)
    assert np.max(np.abs(np.abs(d) - np.abs(dg))) <= 1e-12 * fro
    assert np.max(np.abs(np.abs(e) - np.abs(eg))) <= 1e-12 * fro


@pytest.mark.parametrize("n,bw,tw", [(12, 4, 2), (20, 7, 3), (16, 15, 4)])
def test_singular_values_brute_force_jacobi(n, bw, tw):
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=5)
    A = dense_from_band(band, bw)
    d, e = oracle.reduce(band, bw, tw)
    sb = bidiag_singular_values(d, e)
    sj = jacobi_singular_values(A)
    assert np.max(np.abs(sb - sj)) <= 1e-12 * np.linalg.norm(A)


@pytest.mark.parametrize("n,bw,tw", [(128, 24, 8), (100, 33, 32), (128, 64, 16)])
def test_singular_values_lapack_svd(n, bw, tw):
    band = bb_inputs.make_band(n, bw, "f64", "uniform", seed=7)
    A = dense_from_band(band, bw)
    d, e = oracle.reduce(band, bw, tw)
    B = np.diag(d) + np.diag(e, 1)
    s_ref = np.linalg.svd(A, compute_uv=False)
    s_b = np.linalg.svd(B, compute_uv=False)
    assert np.max(np.abs(s_ref - s_b)) <= 1e-12 * np.linalg.norm(A)


@pytest.mark.parametrize("dt,tol", [("f64", 1e-13), ("f32", 2e-6)])
@pytest.mark.parametrize("n,bw,tw", [(300, 16, 8), (257, 32, 16), (200, 40, 13)])
def test_frobenius_invariance_and_zero_structure(dt, tol, n, bw, tw):
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=11)
    fro2 = np.sum(band.astype(np.float64) ** 2)
    d, e, work, T = oracle.reduce(band, bw, tw, return_band=True)
    got = np.sum(d.astype(np.float64) ** 2) + np.sum(e.astype(np.float64) ** 2)
    assert abs(got - fro2) <= tol * fro2
    assert off_bidiag_max(work, T) == 0.0
    assert np.all(np.isfinite(d)) and np.all(np.isfinite(e))
    np.testing.assert_array_equal(work[:, T], d)
    np.testing.assert_array_equal(work[:-1, T + 1], e)


@pytest.mark.parametrize("n,bw", [(120, 12), (90, 9)])
def test_tile_width_invariance(n, bw):
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=13)
    fro = np.linalg.norm(band)
    d0, e0 = oracle.reduce(band, bw, bw - 1)  # one pass straight to bidiagonal
    for tw in range(1, bw):
        d, e = oracle.reduce(band, bw, tw)
        assert np.max(np.abs(np.abs(d) - np.abs(d0))) <= 1e-12 * fro, tw
        assert np.max(np.abs(np.abs(e) - np.abs(e0))) <= 1e-12 * fro, tw


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_power_of_two_scaling_is_exact(dt):
    n, bw, tw = 150, 20, 6
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=17)
    d, e = oracle.reduce(band, bw, tw)
    # Exact wherever no square underflows; the fp32 tail of the chase sits
    # in denormals (squares ~1e-40) where a scaling shifts the lost bits.
    big = (1e-6 if dt == "f32" else 1e-12) * np.linalg.norm(band.astype(np.float64))
    for s in (0.25, 8.0):
        ds, es = oracle.reduce(band * band.dtype.type(s), bw, tw)
        for got, ref in ((ds, d), (es, e)):
            keep = np.abs(ref) > big
            assert keep.sum() >= len(ref) - 40
            np.testing.assert_array_equal(got[keep], ref[keep] * band.dtype.type(s))
            assert np.all(np.abs(got[~keep]) <= 2 * s * big)


def test_general_scaling_and_negation():
    n, bw, tw = 80, 10, 3
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=19)
    d, e = oracle.reduce(band, bw, tw)
    for s in (-1.0, 3.7, -0.01):
        ds, es = oracle.reduce(band * s, bw, tw)
        assert np.max(np.abs(np.abs(ds) - abs(s) * np.abs(d))) <= 1e-13 * abs(s) * np.linalg.norm(band)
        assert np.max(np.abs(np.abs(es) - abs(s) * np.abs(e))) <= 1e-13 * abs(s) * np.linalg.norm(band)


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_bandwidth_zero_and_one_are_copies(dt):
    n = 37
    b0 = bb_inputs.make_band(n, 0, dt, "normal", seed=1)
    d, e = oracle.reduce(b0, 0, 4)
    np.testing.assert_array_equal(d, b0[:, 0])
    np.testing.assert_array_equal(e, np.zeros(n - 1, dtype=b0.dtype))
    b1 = bb_inputs.make_band(n, 1, dt, "normal", seed=1)
    d, e = oracle.reduce(b1, 1, 4)
    np.testing.assert_array_equal(d, b1[:, 0])
    np.testing.assert_array_equal(e, b1[:-1, 1])


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_all_zero_band(dt):
    n, bw, tw = 64, 16, 8
    band = np.zeros((n, bw + 1), dtype=bb_inputs.np_dtype(dt))
    d, e, work, T = oracle.reduce(band, bw, tw, return_band=True)
    assert np.all(d == 0) and np.all(e == 0)
    assert np.all(work == 0) and np.all(np.isfinite(work))


def test_zero_rows_take_identity_reflectors():
    # rows inside the first b' rows and scattered rows are exactly zero:
    # their row reflectors see a zero tail and must be the identity.
    n, bw, tw = 96, 16, 8
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=23)
    band[[0, 3, 5, 40, 41, 77], :] = 0.0
    A = dense_from_band(band, bw)
    d, e, work, T = oracle.reduce(band, bw, tw, return_band=True)
    assert off_bidiag_max(work, T) == 0.0
    sb = bidiag_singular_values(d, e)
    sa = np.linalg.svd(A, compute_uv=False)
    assert np.max(np.abs(sb - sa)) <= 1e-12 * np.linalg.norm(A)
    assert np.sum(sb <= 1e-12 * np.linalg.norm(A)) >= 6  # structural rank deficiency


@pytest.mark.parametrize("n", [1, 2, 3, 5])
def test_tiny_matrices(n):
    bw, tw = 4, 2
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=29)
    A = dense_from_band(band, bw)
    d, e = oracle.reduce(band, bw, tw)
    assert d.shape == (n,) and e.shape == (max(n - 1, 0),)
    sb = bidiag_singular_values(d, e) if n > 1 else np.abs(d)
    assert np.max(np.abs(sb - np.linalg.svd(A, compute_uv=False))) <= 1e-13 * max(np.linalg.norm(A), 1)


def test_full_upper_triangle_n_le_bw_plus_one():
    # n <= BW+1: the band is the whole upper triangle; every sweep of the
    # first pass has a single cycle (later passes, with smaller b, chase)
    n, bw, tw = 17, 16, 5
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=31)
    b, t = pass_list(bw, tw)[0]
    assert all(cycles_of_sweep(n, b, t, R) == 1 for R in range(n - (b - t) - 1))
    A = dense_from_band(band, bw)
    d, e = oracle.reduce(band, bw, tw)
    dg, eg = dense_golub_kahan(A)
    assert np.max(np.abs(np.abs(d) - np.abs(dg))) <= 1e-12 * np.linalg.norm(A)
    assert np.max(np.abs(np.abs(e) - np.abs(eg))) <= 1e-12 * np.linalg.norm(A)


def test_pass_list_stated_with_the_512_workload():
    w = bb_inputs.WORKLOADS["n512-bw16-tw8-f64-normal"]
    assert [b for b, _ in pass_list(w.bw, w.tw)] + [1] == [16, 8, 1]
    assert pass_list(64, 16) == [(64, 16), (48, 16), (32, 16), (16, 15)]


def test_cycle_count_matches_enumeration():
    n, bw, tw = 200, 24, 7
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=37)
    _, _, done = oracle.reduce(band, bw, tw, max_cycles=10 ** 9)
    assert done == len(sequential_order(n, bw, tw))


def test_three_cycle_separation_keeps_concurrent_cycles_disjoint():
    # Brute force over every step of a one-launch-per-step schedule.
    def conflicts(n, bw, tw, stagger):
        bad = 0
        for (b, t) in pass_list(bw, tw):
            bp = b - t
            nsw = n - bp - 1
            K = [cycles_of_sweep(n, b, t, R) for R in range(nsw)]
            for L in range(max(stagger * R + K[R] for R in range(nsw))):
                seen = set()
                for R in range(nsw):
                    k = L - stagger * R
                    if 0 <= k < K[R]:
                        w = cycle_window(n, b, t, R, k)
                        if seen & w:
                            bad += 1
                        seen |= w
        return bad

    assert conflicts(90, 12, 4, 3) == 0          # b' > 1 and the last pass b' = 1
    assert conflicts(90, 9, 8, 3) == 0           # single pass straight to b' = 1
    assert conflicts(90, 9, 8, 2) > 0            # two cycles fail when b' = 1
    # two cycles suffice for a pass whose target band is wider than bidiagonal
    n, b, t = 90, 12, 4
    for (bb, tt) in [(12, 4), (8, 4)]:
        bp = bb - tt
        nsw = n - bp - 1
        K = [cycles_of_sweep(n, bb, tt, R) for R in range(nsw)]
        for L in range(max(2 * R + K[R] for R in range(nsw))):
            seen = set()
            for R in range(nsw):
                k = L - 2 * R
                if 0 <= k < K[R]:
                    w = cycle_window(n, bb, tt, R, k)
                    assert not (seen & w)
                    seen |= w


@pytest.mark.parametrize("dt", ["f32", "f64"])
@pytest.mark.parametrize("n,bw,tw", [(120, 16, 8), (77, 12, 5), (64, 9, 8)])
def test_staggered_schedules_reproduce_sequential_bits(dt, n, bw, tw):
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=41)
    seq = oracle.run_cycles(band, bw, tw, sequential_order(n, bw, tw))
    _, _, ref, _ = oracle.reduce(band, bw, tw, return_band=True)
    np.testing.assert_array_equal(seq, ref)
    for rev in (True, False):
        st3 = oracle.run_cycles(band, bw, tw, staggered_order(n, bw, tw, 3, rev))
        np.testing.assert_array_equal(st3, ref)


def test_order_violating_dependences_changes_result():
    # A schedule with stagger 1 runs overlapping cycles out of order; the
    # result must differ (shows the schedule test can fail).
    n, bw, tw = 80, 12, 4
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=43)
    _, _, ref, _ = oracle.reduce(band, bw, tw, return_band=True)
    bad = oracle.run_cycles(band, bw, tw, staggered_order(n, bw, tw, 1, True))
    assert not np.array_equal(bad, ref)
