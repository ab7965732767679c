"""Pins for the oracle's decision bands (CPU only).

A coordinate closer to a decision boundary than 1e-6 may take either neighbouring
code, so every band decides which GPU mismatches are forgiven.  Each test builds
an input whose distance to a boundary is known by construction, in the units the
band is defined in, and checks both a case inside the 1e-6 band and one outside
it.  A units slip (a band measured on the unnormalized coordinate, in value units
instead of [0, 1] range units, without the division by 2^b - 1, or a projection
not normalized to a cosine) moves one of these cases across 1e-6 and fails.

Sources: issoh.co.jp "TurboQuantとは？…", 第1段 (Lloyd-Max codes of the rotated
unit vector) and 第2段 (uniform values with a per-vector scale); lilting.ch
TurboQuant article, QJL section (sign bits of a Gaussian projection of the
residual) and PolarQuant section (angles on a uniform grid).
"""
import math

import numpy as np
import pytest

from oracle import tq_oracle as O

BAND = 1e-6
D = 128


def _signs(seed=3):
    rng = np.random.default_rng(seed)
    return np.where(rng.integers(0, 2, D) == 1, 1, -1).astype(np.int8)


def _unit_with(i, value, seed=0):
    """A unit vector of R^128 whose coordinate i is `value` (the others random)."""
    rng = np.random.default_rng(seed)
    y = rng.standard_normal(D)
    y[i] = 0.0
    y *= math.sqrt(1.0 - value * value) / np.linalg.norm(y)
    y[i] = value
    return y


def test_boundary_distance_hand_values():
    t = np.array([-0.25, 0.0, 0.5])
    y = np.array([0.5 + 5e-7, -2e-6, 0.1, -0.2500004])
    assert np.allclose(O.boundary_distance(y, t), [5e-7, 2e-6, 0.1, 4e-7], rtol=1e-9, atol=1e-15)


@pytest.mark.parametrize("mode", ["lloyd", "lloyd_nc"])
@pytest.mark.parametrize("delta", [5e-7, -5e-7, 2e-6, -2e-6])
def test_key_band_in_unit_sphere_units(mode, delta):
    """Rotated unit coordinate t_j + delta: band = |delta| whatever the key's norm."""
    cb = O.codebook(4, D)
    s = _signs()
    j, i = 9, 17                                   # threshold t_9 = 0.2582/sqrt(128) ...
    y = _unit_with(i, cb.thresholds[j] + delta)
    for norm in (1.0, 37.5):
        k = norm * (O.rotation_matrix(s).T @ y)     # R k / ||k|| = y
        kq = O.quantize_keys(k[None], s, cb, mode)
        assert abs(kq.y[0, i] - y[i]) < 1e-14
        assert abs(kq.band[0, i] - abs(delta)) < 1e-12
        assert (kq.band[0, i] < BAND) == (abs(delta) < BAND)
        assert kq.codes[0, i] == (j + 1 if delta > 0 else j)     # code = #{t <= y}


@pytest.mark.parametrize("eps,code", [(7.5e-6, 8), (-7.5e-6, 7), (3e-5, 8), (-3e-5, 7)])
def test_value_band_in_range_units(eps, code):
    """Values in [-4, 4] at 4 bits (scale 8/15): a value whose quotient is 7.5 + eps
    lies eps/15 from the rounding boundary in [0, 1] range units; in value units
    it would be eps * 8/15, without the division by 15 it would be eps."""
    levels = 15
    v = np.full(D, 0.25)
    v[0], v[1] = -4.0, 4.0
    sc = float(np.float32(8.0 / levels))
    v[5] = float(np.float32(-4.0 + sc * (7.5 + eps)))        # an fp32 value, as stored inputs are
    vq = O.quantize_values_uniform(v[None], 4)
    assert vq.vmin[0] == -4.0 and vq.scale[0] == sc
    assert abs(vq.band[0, 5] - abs(eps) / levels) < 1e-8
    assert (vq.band[0, 5] < BAND) == (abs(eps) < 1e-5)
    assert vq.codes[0, 5] == code
    assert vq.codes[0, 0] == 0 and vq.codes[0, 1] == levels


def test_value_band_exact_tie_is_on_the_boundary():
    """Quotient exactly 2.5 at 2 bits: band 0, and round half to even gives 2."""
    v = np.array([[0.0, 3.0, 2.5, 1.5, 0.5]])     # scale 1: quotients 0, 3, 2.5, 1.5, 0.5
    vq = O.quantize_values_uniform(v, 2)
    assert vq.scale[0] == 1.0
    assert np.array_equal(vq.codes[0], [0, 3, 2, 2, 0])
    assert np.all(vq.band[0, 2:] == 0.0)
    assert np.allclose(vq.band[0, :2], 0.5 / 3)


@pytest.mark.parametrize("cos", [5e-7, -5e-7, 2e-6, -2e-6])
def test_qjl_band_is_a_cosine(cos):
    """Row i of S at a known angle to the residual r' (rotated frame): band =
    |cos| whatever the row's length and the key's norm; bit = [cos >= 0]."""
    cb = O.codebook(2, D)
    s = _signs(5)
    rng = np.random.default_rng(11)
    k = 50.0 * rng.standard_normal(D)
    R = O.rotation_matrix(s)
    S = rng.standard_normal((D, D))
    kq = O.quantize_keys(k[None], s, cb, "lloyd_qjl", S)
    # the residual of the stage-1 reconstruction, in the rotated frame
    r = R @ (k - O.dequantize_keys(kq.codes, kq.norm, s, cb)[0])
    rhat = r / np.linalg.norm(r)
    u = rng.standard_normal(D)
    u -= (u @ rhat) * rhat
    u /= np.linalg.norm(u)
    i = 40
    S[i] = 7.0 * (cos * rhat + math.sqrt(1.0 - cos * cos) * u)
    kq = O.quantize_keys(k[None], s, cb, "lloyd_qjl", S)
    assert abs(kq.qjl_band[0, i] - abs(cos)) < 1e-12
    assert (kq.qjl_band[0, i] < BAND) == (abs(cos) < BAND)
    assert kq.qjl_bits[0, i] == (1 if cos > 0 else 0)
    assert abs(kq.qjl_norm[0] - np.linalg.norm(r)) <= 1e-6 * np.linalg.norm(r)


def test_polar_band_in_radians():
    """Level 1 (3 bits, [-pi, pi), cells pi/4 wide, wrapping at +-pi) and level 2
    (3 bits, [0, pi/2], cells pi/16 wide, the range ends are not boundaries)."""
    w1, w2 = math.pi / 4, math.pi / 16
    for theta, code, band in [(-math.pi + w1 + 5e-7, 1, 5e-7), (-math.pi + 3 * w1 - 2e-6, 2, 2e-6),
                              (math.pi - 5e-7, 7, 5e-7), (-math.pi + 5e-7, 0, 5e-7), (0.3, 4, 0.3)]:
        c, b = O.polar_codes(np.array([theta]), 1, 3)
        assert c[0] == code and abs(b[0] - band) < 1e-12, (theta, c, b)
    for theta, code, band in [(3 * w2 + 2e-6, 3, 2e-6), (5 * w2 - 5e-7, 4, 5e-7), (1e-7, 0, w2 - 1e-7),
                              (math.pi / 2 - 1e-7, 7, w2 - 1e-7)]:
        c, b = O.polar_codes(np.array([theta]), 2, 3)
        assert c[0] == code and abs(b[0] - band) < 1e-12, (theta, c, b)


def test_polar_key_band_of_a_known_angle():
    """A rotated vector whose first coordinate pair has angle pi/4 + 4e-7 (a level-1
    edge at 3 bits): the band of that angle's slot is 4e-7 for any key norm."""
    s = _signs(7)
    y = np.random.default_rng(2).standard_normal(D)
    th = math.pi / 4 + 4e-7
    y[0], y[1] = 0.8 * math.cos(th), 0.8 * math.sin(th)
    for norm in (1.0, 20.0):
        k = norm * (O.rotation_matrix(s).T @ y)
        kq = O.quantize_keys_polar(k[None], s, 3)
        slot = O.polar_slot_map(D).index((1, 0))
        assert abs(kq.band[0, slot] - 4e-7) < 1e-12
        assert kq.codes[0, slot] == 5          # [pi/4, pi/2) is cell 5 of [-pi, pi)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_value_band_covers_the_fp32_quotient(bits):
    """The oracle's value codes round the exact quotient (v - min) / scale with the
    stored fp32 min and scale; the kernels round fl32(fl32(v - min) * fl32(1 / scale)).
    Over many vectors of fp32 inputs, including ones placed next to rounding
    boundaries, every code on which the two forms disagree lies inside the value
    band, and some disagreements occur (so the check is not empty)."""
    rng = np.random.default_rng(17 + bits)
    levels = (1 << bits) - 1
    v = rng.standard_normal((4000, D)).astype(np.float32)
    # half of the vectors get coordinates within a few ulps of a rounding boundary
    mn, mx = v.min(axis=1, keepdims=True), v.max(axis=1, keepdims=True)
    sc = ((mx.astype(np.float64) - mn) / levels).astype(np.float32)
    k = rng.integers(0, levels, size=(2000, D))
    near = (mn[:2000] + sc[:2000] * (k + 0.5)).astype(np.float32)
    near = np.nextafter(near, np.where(rng.integers(0, 2, near.shape) == 1, np.inf, -np.inf).astype(np.float32))
    v[:2000, 1:-1] = near[:, 1:-1]
    v[:2000, 0], v[:2000, -1] = mn[:2000, 0], mx[:2000, 0]         # keep the range
    q = O.quantize_values_uniform(v.astype(np.float64), bits)
    vmin, scale = q.vmin.astype(np.float32)[:, None], q.scale.astype(np.float32)[:, None]
    with np.errstate(divide="ignore"):
        inv = np.where(scale > 0, np.float32(1) / scale, np.float32(0)).astype(np.float32)
    prod = ((v - vmin).astype(np.float32) * inv).astype(np.float32)
    fp32_codes = np.clip(np.rint(prod), 0, levels).astype(np.int64)    # rint: half to even
    diff = fp32_codes != q.codes
    assert diff.any(), "no disagreement: the boundary cases did not reach the band"
    assert np.all(q.band[diff] < BAND), q.band[diff].max()
    assert np.all(np.abs(fp32_codes - q.codes) <= 1)
