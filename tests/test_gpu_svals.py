"""Singular values of the bidiagonal by bisection on the GPU (bb_svals,
through the C ABI) against the bisection oracle (needs a GPU).

Both sides follow one reading of page "A two-stage reduction on an Apple M5
Pro", section 7, operation by operation, so the values are compared to the
bit; every bisection depth per round (levels) gives the same bits.  The full
path (band -> bidiagonal -> singular values, all on the GPU) is checked on
the headline-sized band at sampled indices, which the oracle computes one
by one, and against the fp32 accuracy the page states.
"""
import numpy as np
import pytest

import band_bidiagonal_bulge_amd as bbm
import bb_inputs
import oracle
from gpu_util import TOL, assert_bits_equal, gpu_reduce, log

pytestmark = pytest.mark.gpu


def gpu_svals(d, e, i0=0, i1=None, levels=0, tree_levels=0):
    import torch
    dev = torch.device("cuda:0")
    td = torch.from_numpy(np.ascontiguousarray(d)).to(dev)
    te = torch.from_numpy(np.ascontiguousarray(e)).to(dev)
    out = bbm.svals(td, te, i0, i1, levels, tree_levels)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [(1, "normal"), (2, "normal"), (3, "ones"), (64, "normal"), (65, "graded"), (257, "normal"),
         (1000, "graded"), (1500, "ones"), (3001, "normal")]


@pytest.mark.parametrize("dt", ["f32", "f64"])
@pytest.mark.parametrize("n,dist", CASES)
def test_bitwise_equal_to_oracle(n, dist, dt):
    d, e = bb_inputs.make_bidiag(n, dt, dist, seed=n)
    ref = oracle.svals(d, e)
    for (tree, levels) in [(0, 0), (-1, 1), (-1, 2), (-1, 3), (-1, 6), (1, 1), (5, 4), (12, 2), (16, 5)]:
        log(f"svals n={n} {dist} {dt} tree={tree} levels={levels}")
        assert_bits_equal(gpu_svals(d, e, levels=levels, tree_levels=tree), ref)


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_index_ranges_and_ragged_groups(dt):
    n = 777
    d, e = bb_inputs.make_bidiag(n, dt, "normal", seed=5)
    ref = oracle.svals(d, e)
    for (i0, i1, levels, tree) in [(0, 1, 0, 0), (5, 6, 4, -1), (0, 13, 3, 7), (100, 357, 5, 0), (770, 777, 2, 16),
                                   (0, 777, 4, 3), (333, 333, 0, 0)]:
        log(f"svals range {i0}:{i1} {dt} levels={levels} tree={tree}")
        assert_bits_equal(gpu_svals(d, e, i0, i1, levels, tree), ref[i0:i1])


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_degenerate_bidiagonals(dt):
    for (name, d, e) in [("zero", np.zeros(40), np.zeros(39)),
                         ("diag", np.linspace(-3, 2, 50), np.zeros(49)),
                         ("singular", np.r_[np.ones(10), 0.0, np.ones(9)], np.full(19, 0.5)),
                         ("tiny", np.full(30, 1e-30), np.full(29, 3e-31)),
                         ("one", np.array([-2.5]), np.zeros(0))]:
        d, e = d.astype(bb_inputs.np_dtype(dt)), e.astype(bb_inputs.np_dtype(dt))
        log(f"svals degenerate {name} {dt}")
        got = gpu_svals(d, e)
        assert_bits_equal(got, oracle.svals(d, e))
        assert np.all(got >= 0) and not np.any(np.signbit(got))


def test_rejects_bad_calls():
    import torch
    d = torch.ones(8, dtype=torch.float32, device="cuda:0")
    e = torch.ones(7, dtype=torch.float32, device="cuda:0")
    with pytest.raises(bbm.BBError):
        bbm.svals(d, e, 0, 9)
    with pytest.raises(bbm.BBError):
        bbm.svals(d, e, levels=7)
    with pytest.raises(bbm.BBError):
        bbm.svals(d, e, tree_levels=17)
    small = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(bbm.BBError):
        bbm.svals(d, e, work=small)


@pytest.mark.parametrize("dt", ["f32", "f64"])
def test_band_to_singular_values_on_the_gpu(dt):
    # the whole path on the GPU: reduction (bitwise equal to the oracle's d, e
    # elsewhere) then bisection, checked at sampled indices of a 16384 band
    n, bw, tw = 16384, 64, 16
    band = bb_inputs.make_band(n, bw, dt, "normal", seed=0)
    log(f"band->svals n={n} bw={bw} tw={tw} {dt}")
    d, e = gpu_reduce(band, bw, tw)
    sig = gpu_svals(d, e)
    assert np.all(np.diff(sig.astype(np.float64)) <= 0)
    for (i0, i1) in [(0, 48), (8000, 8048), (n - 48, n)]:
        assert_bits_equal(sig[i0:i1], oracle.svals(d, e, i0, i1))
    if dt == "f32":
        # accuracy of the fp32 path against the fp64 path on the same band,
        # within the gate for the fp32 reduction (2e-4 ||A||_F)
        d64, e64 = gpu_reduce(band.astype(np.float64), bw, tw)
        ref = oracle.svals(d64, e64, 0, 48)
        err = float(np.max(np.abs(sig[:48] - ref)))
        log(f"fp32 vs fp64 path: max |dsigma| / sigma_max = {err / ref[0]:.3e}")
        assert err <= TOL["f32"] * np.linalg.norm(band.astype(np.float64))
