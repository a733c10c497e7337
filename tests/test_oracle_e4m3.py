"""Pins of the oracle's OCP E4M3 codec against the format's definition.

E4M3 (the OCP 8-bit floating point format, E4M3 variant) is the FP8 format of
V and P in the method; the decode values below are fixed by the format: sign,
4-bit exponent with bias 7, 3-bit mantissa, exponent field 0 subnormal, only
S.1111.111 NaN, largest finite 448.
"""
import math

import numpy as np
import pytest

import oracle


def test_decode_fixed_points():
    dec = oracle.e4m3_decode(np.arange(256))
    assert dec[0x7E] == 448.0
    assert dec[0xFE] == -448.0
    assert dec[0x38] == 1.0
    assert dec[0x30] == 0.5
    assert dec[0x08] == 2.0 ** -6          # smallest normal
    assert dec[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert dec[0x01] == 2.0 ** -9          # smallest subnormal
    assert dec[0x77] == 240.0
    assert dec[0x00] == 0.0 and not math.copysign(1.0, dec[0x00]) < 0
    assert dec[0x80] == 0.0 and math.copysign(1.0, dec[0x80]) < 0
    assert math.isnan(dec[0x7F]) and math.isnan(dec[0xFF])
    finite = dec[:0x7F]
    assert np.all(np.diff(finite) > 0), "codes must be monotone in magnitude"
    assert np.array_equal(dec[0x80:0xFF], -dec[0x00:0x7F])
    assert len(set(dec[~np.isnan(dec)].tolist())) == 253


def test_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),          # midpoint of 1 and 1.125 -> even mantissa 0
    (1.1875, 0x3A),          # midpoint of 1.125 and 1.25 -> even mantissa 2
    (2.0 ** -10, 0x00),      # midpoint of 0 and 2^-9 -> 0
    (-(2.0 ** -10), 0x80),   # sign of zero kept
    (1.5 * 2.0 ** -9, 0x02), # midpoint of 1 and 2 subnormal steps -> 2
    (0.75 * 2.0 ** -9, 0x01),
    (15.5 * 2.0 ** -10, 0x08),  # 7.75 * 2^-9 rounds up into the smallest normal
    (440.0, 0x7E),           # midpoint of 416 and 448 -> even mantissa 6 (448)
    (432.0, 0x7E),
    (431.99, 0x7D),
    (1e-8, 0x00),
    (-1e-8, 0x80),
    (0.013671875, 0x07),
])
def test_ties_and_edges(x, code):
    assert oracle.e4m3_encode(np.array([x], np.float32))[0] == code
    assert oracle.e4m3_encode_nearest(x) == code


def test_structured_sweep_agrees_with_nearest_search():
    # every sign/exponent/top-7-mantissa pattern with low 16 bits at and around
    # the rounding cut positions; the cut of every E4M3 result lies in the top
    # 16 bits of the FP32 word
    lows = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000]
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    bits = (hi[:, None] | np.array(lows, dtype=np.uint32)[None, :]).ravel()
    x = bits.view(np.float32)
    x = x[np.abs(x) <= 448.0]
    got = oracle.e4m3_encode(x)
    sample = x[:: max(1, x.size // 4000)]
    ref = np.array([oracle.e4m3_encode_nearest(float(v)) for v in sample], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(sample), ref)
    assert got.shape == x.shape


@pytest.mark.slow
def test_exhaustive_sweep_two_encoders():
    # all 2^32 FP32 patterns with |x| <= 448: arithmetic encoder vs nearest
    # search over the sorted code table with ties to the even code
    assert oracle.e4m3_sweep_mismatches(0, 1 << 31) == 0
    assert oracle.e4m3_sweep_mismatches(1 << 31, (1 << 32) - 1) == 0
