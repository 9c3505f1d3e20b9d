"""The seeded input generators: shapes, seeds, and the known-spectrum bands
of the accuracy study (their singular values are the prescribed ones)."""
import numpy as np
import pytest

import bb_inputs


@pytest.mark.parametrize("spectrum", bb_inputs.SPECTRA)
def test_known_spectrum_band_has_the_prescribed_singular_values(spectrum):
    n, bw = 160, 16
    band, sigma = bb_inputs.known_spectrum_band(n, bw, spectrum, seed=4)
    assert band.shape == (n, bw + 1)
    assert np.all(np.diff(sigma) <= 0) and sigma[0] <= 1 and sigma[-1] >= 0
    A = np.zeros((n, n))
    for o in range(bw + 1):
        A[np.arange(n - o), np.arange(n - o) + o] = band[:n - o, o]
    sv = np.linalg.svd(A, compute_uv=False)
    assert np.linalg.norm(sv - sigma) <= 1e-13 * np.linalg.norm(sigma)


def test_spectra():
    rng = np.random.default_rng(0)
    a = bb_inputs.known_spectrum(100, "arithmetic", rng)
    assert a[0] == 1.0 and np.allclose(np.diff(a), -0.01)
    g = bb_inputs.known_spectrum(100, "logarithmic", rng)
    assert g[0] == 1.0 and np.isclose(g[-1], 1e-6) and np.allclose(np.diff(np.log10(g)), -6 / 99)
    q = bb_inputs.known_spectrum(20000, "quarter_circle", rng)
    # quarter-circle law on [0, 1]: mean 4/(3 pi)
    assert abs(np.mean(q) - 4 / (3 * np.pi)) < 0.01


def test_seeds_reproduce():
    a = bb_inputs.make_band(50, 5, "f32", "normal", seed=3)
    b = bb_inputs.make_band(50, 5, "f32", "normal", seed=3)
    assert np.array_equal(a, b)
    assert bb_inputs.make_band(10, 2, "f16", "normal").dtype == np.float16
