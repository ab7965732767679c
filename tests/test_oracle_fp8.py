"""Pins of the oracle's FP8 (E4M3) key path (issoh.co.jp "TurboQuantとは？…",
preset table: one serving preset stores the keys in FP8 and the values in 4 bits).

* the code table against the closed form of the format (named values, order,
  symmetry, the NaN codes);
* rounding against an independent library routine: torch's float32 ->
  float8_e4m3fn cast, for every finite bf16 value of magnitude at most 448;
* ties to the even code on the midpoints; saturation above 448 (reading R24);
* round trip of every finite code; the page layout of the preset (200 bytes per
  token-head with 4-bit uniform values, the 2.6x of the preset table).
"""
import numpy as np
import pytest

from oracle import tq_oracle as O

torch = pytest.importorskip("torch")


def test_code_table_closed_form():
    v = O.fp8_e4m3_value(np.arange(256))
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6                   # smallest normal
    assert v[0x38] == 1.0 and v[0x39] == 1.125 and v[0x37] == 0.9375
    assert v[0x7E] == 448.0 and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)               # codes 0..126 increase
    assert np.array_equal(v[0x80:0xFF], -pos)     # the sign bit mirrors them


def test_rounding_matches_torch_cast_on_every_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    keep = np.isfinite(x) & (np.abs(x) <= 448.0)
    x = x[keep]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    got = O.quantize_fp8_e4m3(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_ties_go_to_the_even_code():
    v = O.fp8_e4m3_value(np.arange(0x7F))
    mid = (v[:-1] + v[1:]) / 2                    # exact in fp64
    got = O.quantize_fp8_e4m3(mid)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    assert np.array_equal(O.quantize_fp8_e4m3(-mid), got | 0x80)


def test_saturation_and_signed_zero():
    assert list(O.quantize_fp8_e4m3([448.0, 460.0, 1e6, -500.0])) == [0x7E, 0x7E, 0x7E, 0xFE]
    assert list(O.quantize_fp8_e4m3([0.0, -0.0, 2.0 ** -11, -2.0 ** -11])) == [0x00, 0x80, 0x00, 0x80]


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(O.quantize_fp8_e4m3(O.fp8_e4m3_value(codes)), codes)


def test_fp8_key_layout_and_reconstruction():
    cfg = O.Config(128, 2, 8, 8, "fp8", 4, "uniform")
    f = O.page_fields(cfg)
    assert "knorm" not in f and f["kcodes"] == (0, 128)
    assert O.page_bytes(cfg) == 16 * 200 and 512 / 200 == pytest.approx(2.56)
    rng = np.random.default_rng(3)
    k = rng.standard_normal((40, 2, 128)) * 3.0
    v = rng.standard_normal((40, 2, 128))
    cache = O.new_cache(cfg, 4)
    slots = np.arange(40) + 8
    O.quantize_append(cfg, cache, k, v, slots, np.ones(128), O.codebook(4, 128))
    for h in range(2):
        kh, vh, f = O.dequantize_slots(cfg, cache, slots, h, np.ones(128), O.codebook(4, 128), None)
        assert np.array_equal(kh, O.fp8_e4m3_value(O.quantize_fp8_e4m3(k[:, h])))
        # relative error of E4M3 is at most 2^-4 for normal values
        big = np.abs(k[:, h]) >= 2.0 ** -6
        assert np.all(np.abs(kh - k[:, h])[big] <= 2.0 ** -4 * np.abs(k[:, h])[big])
