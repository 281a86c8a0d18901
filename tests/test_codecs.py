"""Pins of the oracle's rounding functions against library codecs and the format definitions."""
import numpy as np
import pytest
import torch

from oracle.codecs import bf16, e4m3, e4m3_decode, e4m3_encode, fl32, rne


def test_e4m3_all_codes_round_trip():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_decode(codes)
    finite = ~np.isnan(vals)
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF]) and finite.sum() == 254
    assert np.array_equal(e4m3(vals[finite]), vals[finite])
    assert np.array_equal(e4m3_encode(vals[finite]), codes[finite])


def test_e4m3_format_extremes():
    # largest finite 448 = 1.75 * 2^8 is code 0x7E; smallest subnormal 2^-9 is 0x01
    assert e4m3_decode(np.array([0x7E, 0x01, 0x08, 0x80]))[:3].tolist() == [448.0, 2.0 ** -9, 2.0 ** -6]
    assert np.signbit(e4m3_decode(np.array([0x80])))[0]


@pytest.mark.parametrize("x,want", [
    (1.0625, 1.0),          # midpoint of 1 and 1.125 goes to the even mantissa
    (1.1875, 1.25),         # midpoint of 1.125 and 1.25 goes to the even mantissa
    (464.0, 448.0),         # midpoint of 448 and 480 goes to 448 (even)
    (470.0, 448.0),         # above the largest finite: saturates
    (1e6, 448.0),
    (-1e6, -448.0),
    (2.0 ** -10, 0.0),      # half the smallest subnormal ties to zero
    (1.5 * 2.0 ** -10, 2.0 ** -9),
    (3.0 * 2.0 ** -10, 2.0 ** -8),  # 1.5 subnormal steps ties to 2 steps
    (15 * 2.0 ** -10, 2.0 ** -6),   # 7.5 subnormal steps ties to the smallest normal
])
def test_e4m3_rounding_cases(x, want):
    assert e4m3(np.array([x]))[0] == want


def test_e4m3_matches_torch_float8_e4m3fn():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 30,
        rng.uniform(-464, 464, 20000),
        rng.standard_normal(20000) * 2.0 ** -7,
        # every midpoint between neighbouring finite codes
        (lambda v: (v[:-1] + v[1:]) / 2)(np.sort(e4m3_decode(np.arange(0, 0x7F)))),
    ]).astype(np.float32)
    x = x[np.abs(x) <= 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(e4m3(x.astype(np.float64)), ref)


def test_bf16_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000),
                        rng.standard_normal(1000) * 1e-39]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16(x.astype(np.float64)), ref)
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1)
    assert bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8]))[:].tolist() == [1.0, 1 + 2.0 ** -6]
    assert np.isinf(bf16(np.array([3.4e38]))[0])


def test_fl32_ties_and_int8_rounding():
    assert fl32(np.array([1 + 2.0 ** -24]))[0] == 1.0
    assert fl32(np.array([1 + 3 * 2.0 ** -24]))[0] == 1 + 2.0 ** -22
    v = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5])
    assert rne(v).tolist() == [0.0, 2.0, 2.0, -0.0, -2.0, -2.0, 126.0]
    assert np.array_equal(rne(v), np.array([round(t) for t in v], dtype=np.float64))
