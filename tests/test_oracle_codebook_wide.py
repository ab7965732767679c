"""Pins of the oracle's Lloyd-Max codebooks with many levels (5 to 8 bits; the
8-bit key preset: issoh.co.jp "TurboQuantとは？…", the MLX section names a
default with 8-bit keys and 3-bit values).  The alternation of the two
optimality conditions converges slowly with many levels, so the oracle finishes
with Newton's method; these checks use only the definition:

* fixpoint: every centroid is the mean of N(0,1) over its cell and every
  threshold the midpoint of its neighbours (cell masses from scipy's normal CDF,
  not from the oracle's tail function);
* symmetry and order;
* distortion: computed in closed form per cell, it decreases by about 4x per
  bit and approaches the high-resolution (Panter-Dite) value
  sqrt(3) pi / 2 * 4^-b from below, within 1% at 8 bits.
"""
import math

import numpy as np
import pytest
from scipy.special import ndtr

from oracle import tq_oracle as O


def _phi(x):
    x = np.asarray(x, np.float64)
    fin = np.isfinite(x)
    return np.where(fin, np.exp(-0.5 * np.where(fin, x, 0.0) ** 2) / math.sqrt(2 * math.pi), 0.0)


def _cells(c, t):
    e = np.concatenate([[-np.inf], t, [np.inf]])
    return e[:-1], e[1:]


def _mass(a, b):
    """P(a < Z < b), from the tail on the cell's side (no cancellation far out)."""
    return np.where(a >= 0, ndtr(-a) - ndtr(-b), ndtr(b) - ndtr(a))


@pytest.mark.parametrize("bits", [5, 6, 8])
def test_wide_codebook_is_a_lloyd_max_fixpoint(bits):
    c, t = O.lloyd_max_standard_normal(bits)
    assert c.shape == (1 << bits,) and t.shape == ((1 << bits) - 1,)
    a, b = _cells(c, t)
    mass = _mass(a, b)
    mean = (_phi(a) - _phi(b)) / mass
    assert np.max(np.abs(mean - c)) < 1e-12
    assert np.max(np.abs(t - 0.5 * (c[:-1] + c[1:]))) < 1e-15
    assert np.all(np.diff(c) > 0) and np.allclose(c, -c[::-1], atol=0, rtol=0)
    assert t[len(t) // 2] == 0.0


def test_distortion_approaches_the_high_resolution_limit():
    ratios = []
    for bits in range(2, 9):
        c, t = O.lloyd_max_standard_normal(bits)
        a, b = _cells(c, t)
        mass = _mass(a, b)
        m1 = _phi(a) - _phi(b)
        m2 = mass + np.where(np.isfinite(a), a, 0.0) * _phi(a) - np.where(np.isfinite(b), b, 0.0) * _phi(b)
        dist = float(np.sum(m2 - 2 * c * m1 + c * c * mass))
        ratios.append(dist / (math.sqrt(3) * math.pi / 2 * 4.0 ** -bits))
    assert abs(ratios[0] * (math.sqrt(3) * math.pi / 2 / 16) - 0.117482) < 1e-5   # textbook 2-bit value
    assert all(r2 > r1 for r1, r2 in zip(ratios, ratios[1:]))
    assert 0.99 < ratios[-1] < 1.0
