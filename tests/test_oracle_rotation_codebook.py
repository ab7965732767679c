"""Pins for the oracle's rotation and Lloyd-Max codebook (CPU only).

Rotation: issoh.co.jp TurboQuant page, stage-1 section (random rotation) and the
llama.cpp Hadamard section (normalized Walsh-Hadamard transform).
Codebook: same page, stage-1 section (per-coordinate Lloyd-Max), checked against
Max (1960) and against independent quadrature of the optimality conditions.
"""
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import scipy.stats

from oracle import tq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_orthogonality_exact(d):
    h = O.hadamard(d)
    assert np.array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))


@pytest.mark.parametrize("d", [2, 4, 64, 128])
def test_hadamard_matches_library_and_closed_form(d):
    h = O.hadamard(d)
    assert np.array_equal(h, scipy.linalg.hadamard(d))
    i = np.arange(d)
    pop = np.vectorize(lambda x: bin(x).count("1"))(i[:, None] & i[None, :])
    assert np.array_equal(h, (-1) ** pop)           # H_ij = (-1)^popcount(i & j)


def test_rotation_hand_example_d4():
    # s = [1,-1,1,1], x = [1,2,3,4]: s*x = [1,-2,3,4]; H4 (s*x) = [6,2,-8,4]; / sqrt(4)
    r = O.rotation_matrix(np.array([1, -1, 1, 1]))
    assert np.allclose(r @ np.array([1.0, 2, 3, 4]), [3.0, 1.0, -4.0, 2.0], atol=1e-15)


def test_rotation_orthogonal_and_columns():
    rng = np.random.default_rng(0)
    s = np.where(rng.integers(0, 2, 128) == 1, 1, -1)
    r = O.rotation_matrix(s)
    assert np.abs(r @ r.T - np.eye(128)).max() < 1e-13
    x = rng.standard_normal((50, 128))
    assert np.allclose(np.linalg.norm(x @ r.T, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # R e_i is column i: s_i * H[:, i] / sqrt(d)
    h = scipy.linalg.hadamard(128)
    for i in (0, 5, 77, 127):
        e = np.zeros(128)
        e[i] = 1.0
        assert np.allclose(r @ e, s[i] * h[:, i] / math.sqrt(128), atol=1e-15)


def _load_max_table():
    rows = {}
    with open(os.path.join(GOLDEN, "lloyd_max_gaussian.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            b, c, t, dist = [p.strip() for p in line.split("|")]
            rows[int(b)] = ([float(x) for x in c.split()], [float(x) for x in t.split()], float(dist))
    return rows


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_matches_max_1960(bits):
    c_ref, t_ref, _ = _load_max_table()[bits]
    c, t = O.lloyd_max_standard_normal(bits)
    assert np.allclose(c[len(c) // 2:], c_ref, atol=6e-4, rtol=5e-4)
    assert np.allclose(t[len(t) // 2 + 1:], t_ref, atol=6e-4, rtol=5e-4)
    assert t[len(t) // 2] == 0.0


def test_lloyd_max_one_bit_closed_form():
    c, t = O.lloyd_max_standard_normal(1)
    assert np.allclose(c, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], rtol=1e-14)
    assert np.array_equal(t, [0.0])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_max_optimality_by_quadrature(bits):
    """Centroid condition checked with scipy quadrature (independent of the solver's formula);
    midpoint condition exact; distortion equals Max's printed value."""
    c, t = O.lloyd_max_standard_normal(bits)
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    pdf = scipy.stats.norm.pdf
    dist = 0.0
    for i in range(len(c)):
        a, b = edges[i], edges[i + 1]
        mass = scipy.integrate.quad(pdf, a, b, epsabs=1e-15, epsrel=1e-13)[0]
        mean = scipy.integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-15, epsrel=1e-13)[0] / mass
        assert abs(mean - c[i]) < 1e-10
        dist += scipy.integrate.quad(lambda x: (x - c[i]) ** 2 * pdf(x), a, b, epsabs=1e-15, epsrel=1e-12)[0]
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-15)
    assert np.allclose(c, -c[::-1], atol=0)
    assert abs(dist - _load_max_table()[bits][2]) / dist < 2e-3


def test_codebook_scales_with_head_dim():
    cb = O.codebook(4, 128)
    c, t = O.lloyd_max_standard_normal(4)
    assert np.allclose(cb.centroids * math.sqrt(128), c, rtol=1e-15)
    assert np.allclose(cb.thresholds * math.sqrt(128), t, rtol=1e-15)
