"""Pins of the oracle's fp8 e4m3fn cache format.

The cache write multiplies a bf16 value by the fp32 reciprocal of the
per-tensor scale and rounds to e4m3fn with saturation.  The reference here is
a brute-force nearest-value search over every finite e4m3fn code (values
decoded by the independent pure-Python decoder), with ties to the even code,
run over all 65,536 bf16 bit patterns.
"""
import numpy as np
import pytest

import oracle
from oracle import brute

POS_CODES = np.arange(0x7F, dtype=np.uint8)  # 0x00 .. 0x7E: every finite non-negative code
POS_VALUES = np.array([brute.e4m3fn_to_float(int(c)) for c in POS_CODES], dtype=np.float64)


def nearest_code(y: np.ndarray) -> np.ndarray:
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    sign = np.signbit(y).astype(np.uint8) << 7
    hi = np.searchsorted(POS_VALUES, a, side="left").clip(0, len(POS_VALUES) - 1)
    lo = (hi - 1).clip(0, None)
    d_lo = np.abs(a - POS_VALUES[lo])
    d_hi = np.abs(POS_VALUES[hi] - a)
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = POS_CODES[pick]
    code = np.where(a >= 448.0, np.uint8(0x7E), code)  # saturation
    out = (code | sign).astype(np.uint8)
    return np.where(np.isnan(y), np.uint8(0x7F), out)


def test_format_values_from_definition():
    assert brute.e4m3fn_to_float(0x7E) == 448.0
    assert brute.e4m3fn_to_float(0x38) == 1.0
    assert brute.e4m3fn_to_float(0x08) == 2.0 ** -6
    assert brute.e4m3fn_to_float(0x01) == 2.0 ** -9
    assert brute.e4m3fn_to_float(0xB8) == -1.0
    assert np.isnan(brute.e4m3fn_to_float(0x7F)) and np.isnan(brute.e4m3fn_to_float(0xFF))
    # the C oracle decodes every code to the same value
    for c in range(256):
        a, b = oracle.fp8_value([c])[0], brute.e4m3fn_to_float(c)
        assert (np.isnan(a) and np.isnan(b)) or a == b


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = np.array([brute.e4m3fn_to_float(int(c)) for c in codes], dtype=np.float32)
    assert np.array_equal(oracle.fp8_encode(vals), codes)


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -4, float(np.float32(5.3 / 448.0)), 0.0131, 3.7, 1e-3])
def test_exhaustive_bf16_quantisation(scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    inv = np.float32(1.0) / np.float32(scale)
    y = (x * inv).astype(np.float32)
    expect = nearest_code(y)
    got = oracle.fp8_quantize(bits, scale)
    bad = np.nonzero(got != expect)[0]
    assert bad.size == 0, [(hex(int(bits[i])), float(y[i]), hex(int(got[i])), hex(int(expect[i])))
                           for i in bad[:8]]


def test_saturation_and_midpoints():
    cases = {448.0: 0x7E, 500.0: 0x7E, 1e30: 0x7E, -1e30: 0xFE, np.inf: 0x7E,
             1.0625: 0x38,  # midway between 1.0 (m=0) and 1.125 (m=1): even code
             1.1875: 0x3A,  # midway between 1.125 (m=1) and 1.25 (m=2): even code
             2.0 ** -10: 0x00,  # half the smallest subnormal ties to zero
             3 * 2.0 ** -10: 0x02,  # 1.5 quanta ties to the even code 2
             -0.0: 0x80}
    ys = np.array(list(cases.keys()), dtype=np.float32)
    assert [hex(c) for c in oracle.fp8_encode(ys)] == [hex(c) for c in cases.values()]
