"""The threaded CPU chaser (the oracle's cycles with the sweeps of a pass on
host threads, page "A two-stage reduction on an Apple M5 Pro", section 6)
against the sequential oracle: same d, e and working band to the bit, for
every thread count, both precisions, bidiagonal (b' = 1) and wider targets,
tiny and ragged shapes.  A stopped-early run (first pass only) equals the
sequential oracle's cycles of that pass, run in order.
"""
import numpy as np
import pytest

import bb_inputs
import oracle
from refs import cycles_of_sweep, pass_list

SHAPES = [(1, 0, 1), (2, 1, 1), (5, 4, 3), (40, 6, 2), (64, 16, 8), (100, 9, 4), (33, 32, 16),
          (50, 12, 1), (130, 17, 16), (257, 32, 16), (300, 5, 3), (96, 2, 1)]


@pytest.mark.parametrize("n,bw,tw", SHAPES)
@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_threaded_equals_sequential(n, bw, tw, dtype):
    band = bb_inputs.make_band(n, bw, dtype, "normal", seed=n + bw)
    d, e, W, T = oracle.reduce(band, bw, tw, return_band=True)
    for threads in (1, 2, 3, 8):
        d2, e2, W2, T2, used = oracle.reduce_mt(band, bw, tw, threads=threads, return_band=True)
        assert T2 == T
        assert used <= threads
        assert np.array_equal(W2, W), (threads, dtype)
        assert np.array_equal(d2, d) and np.array_equal(e2, e)


@pytest.mark.parametrize("dist", ["uniform_zero_rows", "graded"])
def test_threaded_structured_inputs(dist):
    n, bw, tw = 200, 24, 8
    band = bb_inputs.make_band(n, bw, "f32", dist, seed=7)
    d, e = oracle.reduce(band, bw, tw)
    d2, e2, _ = oracle.reduce_mt(band, bw, tw, threads=5)
    assert np.array_equal(d2, d) and np.array_equal(e2, e)


def test_threaded_mixed_precision():
    n, bw, tw = 150, 20, 6
    band = bb_inputs.make_band(n, bw, "f32", "normal", seed=2)
    d, e = oracle.reduce(band, bw, tw, compute="f64")
    d2, e2, _ = oracle.reduce_mt(band, bw, tw, threads=4, compute="f64")
    assert d2.dtype == np.float64
    assert np.array_equal(d2, d) and np.array_equal(e2, e)


def test_first_pass_only_equals_its_cycles_in_order():
    n, bw, tw = 180, 24, 8
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=11)
    b, t = pass_list(bw, tw)[0]
    order = [(0, R, k) for R in range(n - (b - t) - 1) for k in range(cycles_of_sweep(n, b, t, R))]
    ref = oracle.run_cycles(band, bw, tw, order)
    _, _, W, _, _ = oracle.reduce_mt(band, bw, tw, threads=6, return_band=True, max_passes=1)
    assert np.array_equal(W, ref)


def test_threads_capped_by_sweeps():
    n, bw, tw = 12, 8, 4        # passes 8 -> 4 -> 1: 7 and 10 sweeps
    band = bb_inputs.make_band(n, bw, "f64", "normal", seed=0)
    _, _, used = oracle.reduce_mt(band, bw, tw, threads=64)
    assert used == max(n - (b - t) - 1 for (b, t) in pass_list(bw, tw)) == 10
    _, _, used = oracle.reduce_mt(band, bw, tw, threads=64, max_passes=1)
    assert used == 7


def test_rejects_bad_arguments():
    band = bb_inputs.make_band(16, 4, "f64", "normal", seed=0)
    with pytest.raises(ValueError):
        oracle.reduce_mt(band, 4, 0)
    with pytest.raises(ValueError):
        oracle.reduce_mt(band[:, :3], 4, 2)


def test_page_thread_caps():
    # negative counts take the page's caps: at most 2n/(3b) and n/256 threads
    n, bw, tw = 1024, 64, 32                     # passes 64 -> 32 -> 1
    band = bb_inputs.make_band(n, bw, "f32", "normal", seed=4)
    d, e = oracle.reduce(band, bw, tw)
    d2, e2, used = oracle.reduce_mt(band, bw, tw, threads=-16, max_passes=1)
    assert used == min(16, 2 * n // (3 * 64), n // 256) == 4
    d2, e2, used = oracle.reduce_mt(band, bw, tw, threads=-16)
    assert used == 4 and np.array_equal(d2, d) and np.array_equal(e2, e)
    _, _, used = oracle.reduce_mt(band[:200], bw, tw, threads=-16)
    assert used == 1
