"""Pins of the fp16 oracle (the oracle's body instantiated on an emulated
IEEE binary16 type; page "Accelerating Bidiagonalization of Banded Matrices
through Memory-Aware Bulge-Chasing on GPUs", the FP16 variant run in the
accuracy study) to facts other than itself:
  * conversions: every one of the 65536 bit patterns decodes as numpy's
    float16 does, and rounding doubles to binary16 matches numpy's cast
    (ties to even, subnormals, overflow);
  * fma, division and square root are correctly rounded: compared with the
    exact rational result rounded to nearest-even by a rounding written here
    with fractions, on random operands and on constructed ties;
  * the reduction: |d|, |e| against the fp64 oracle within the fp16 error
    level, exact zeros off the bidiagonal, identity reflectors on zero rows.
The reduction steps themselves are the fp32/fp64 oracle's body text, pinned
in test_oracle_pins.py and test_oracle_mutants.py.
"""
from fractions import Fraction

import numpy as np
import pytest

import bb_inputs
import oracle


def round_h16(q: Fraction) -> float:
    """Exact rational -> nearest binary16 (ties to even), as a float."""
    if q == 0:
        return 0.0
    s = -1.0 if q < 0 else 1.0
    a = abs(q)
    if a >= Fraction(65520):
        return s * float("inf")
    e = -14
    if a >= Fraction(2) ** -14:
        e = a.numerator.bit_length() - a.denominator.bit_length()
        while Fraction(2) ** e > a:
            e -= 1
        while Fraction(2) ** (e + 1) <= a:
            e += 1
    ulp = Fraction(2) ** (e - 10)
    k = a / ulp
    n = k.numerator // k.denominator
    rem = k - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return s * float(n * ulp)


def h(x):
    return int(np.float16(x).view(np.uint16))


def hv(b):
    return float(np.uint16(b).view(np.float16))


def test_all_bit_patterns_decode():
    L = oracle.f16_lib()
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    mine = np.array([L.bb_oracle_h16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_rounding_to_binary16():
    L = oracle.f16_lib()
    rng = np.random.default_rng(0)
    xs = rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 5, 20000)
    edges = [65519.99, 65520.0, 65504.0, 2.0 ** -25, 3 * 2.0 ** -26, 1.5 * 2.0 ** -24, 2.0 ** -26, 0.0, -0.0,
             1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2048.5, -65520.0]
    xs = np.concatenate([xs, edges])
    mine = np.array([L.bb_oracle_h16_from_double(float(x)) for x in xs], dtype=np.uint16)
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)


def _random_halves(rng, k):
    mags = 2.0 ** rng.integers(-26, 14, k) * rng.uniform(1, 2, k)
    return np.where(rng.random(k) < 0.5, -1, 1) * mags


def test_fma_division_sqrt_correctly_rounded():
    L = oracle.f16_lib()
    rng = np.random.default_rng(1)
    a, b, c = (_random_halves(rng, 3000) for _ in range(3))
    for x, y, z in zip(a, b, c):
        hx, hy, hz = h(x), h(y), h(z)
        X, Y, Z = (Fraction(hv(v)) for v in (hx, hy, hz))
        if not all(np.isfinite([hv(hx), hv(hy), hv(hz)])):
            continue
        assert hv(L.bb_oracle_h16_fma(hx, hy, hz)) == round_h16(X * Y + Z)
        if Y != 0:
            assert hv(L.bb_oracle_h16_div(hx, hy)) == round_h16(X / Y)
        if X >= 0:
            r = hv(L.bb_oracle_h16_sqrt(hx))
            # r is the correctly rounded square root: compare squares exactly
            lo, hi = np.nextafter(np.float16(r), np.float16(0)), np.nextafter(np.float16(r), np.float16(np.inf))
            R = Fraction(r)
            if r > 0:
                assert (Fraction(float(lo)) + R) ** 2 <= 4 * X <= (R + Fraction(float(hi))) ** 2


def test_fma_ties_go_by_the_exact_value():
    L = oracle.f16_lib()
    # a*b + c landing exactly halfway between two halves after one rounding
    # of the sum, with a tiny remainder on either side
    one = h(1.0)
    for (x, y, z) in [(1.0, 1.0, 2.0 ** -11), (1 + 2.0 ** -10, 1 + 2.0 ** -10, -1.0), (3.0, 2.0 ** -12, 1.0),
                      (1 + 2.0 ** -10, 2.0 ** -11, 1.0), (-(1 + 2.0 ** -10), 2.0 ** -11, 1.0)]:
        X, Y, Z = Fraction(hv(h(x))), Fraction(hv(h(y))), Fraction(hv(h(z)))
        assert hv(L.bb_oracle_h16_fma(h(x), h(y), h(z))) == round_h16(X * Y + Z), (x, y, z)
    assert one == 0x3C00


@pytest.mark.parametrize("n,bw,tw", [(128, 16, 8), (200, 9, 4), (64, 32, 31), (300, 24, 5)])
def test_reduction_against_fp64(n, bw, tw):
    band = bb_inputs.make_band(n, bw, "f16", "normal", seed=n)
    d, e, W, T = oracle.reduce(band, bw, tw, return_band=True)
    assert d.dtype == np.float16
    d64, e64 = oracle.reduce(band.astype(np.float64), bw, tw)
    fro = np.linalg.norm(band.astype(np.float64))
    assert np.max(np.abs(np.abs(d.astype(np.float64)) - np.abs(d64))) <= 0.05 * fro
    assert np.max(np.abs(np.abs(e.astype(np.float64)) - np.abs(e64))) <= 0.05 * fro
    off = [o for o in range(W.shape[1]) if o - T not in (0, 1)]
    assert np.all(W[:, off] == 0)


def test_zero_rows_and_bidiagonal_input():
    band = bb_inputs.make_band(120, 8, "f16", "uniform_zero_rows", seed=2)
    d, e = oracle.reduce(band, 8, 3)
    assert np.all(np.isfinite(d)) and np.all(np.isfinite(e))
    band = bb_inputs.make_band(50, 1, "f16", "normal", seed=3)
    d, e = oracle.reduce(band, 1, 4)
    np.testing.assert_array_equal(d, band[:, 0])
    np.testing.assert_array_equal(e, band[:-1, 1])
