"""Pins for the constants the device decode uses in place of a division.

The kernels compute the code value RN_f32(y / d) (d = 147.800537109375, the
divisor of the pages' value helpers: mlx-bun 0.2.0 -> 0.4.0 diff, page 55,
trellis-linear.ts HEADER, trellis_val) as one fused operation
fma(y, r_hi, RN_f32(y * r_lo)) with r_hi = RN_f32(1/d) and r_lo the binary32
literal kRcpLo in csrc/trellis_device.hpp.  These tests read the constants
from that header and check, in exact rational arithmetic, that the result is
the correctly rounded quotient for every code y in [-510, 510].
"""
import os
import re
from fractions import Fraction

import numpy as np

HDR = os.path.join(os.path.dirname(__file__), "..", "trellis_coded_quantized_amd", "csrc",
                   "trellis_device.hpp")


def _constants():
    text = open(HDR).read()
    d = re.search(r"kDiv\s*=\s*([0-9.]+)f;", text).group(1)
    lo = re.search(r"kRcpLo\s*=\s*(-?0x[0-9a-fA-F.]+p-?[0-9]+)f;", text).group(1)
    return Fraction(d), np.float32(float.fromhex(lo))


def _rn32(q: Fraction) -> np.float32:
    """Round a rational to the nearest binary32, ties to even."""
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - q), int(np.float32(c).view(np.uint32)) & 1))


def test_divisor_is_exact_binary32():
    d, _ = _constants()
    assert Fraction(float(np.float32(float(d)))) == d == Fraction(605391, 4096)


def test_low_part_is_the_rounded_remainder():
    d, lo = _constants()
    hi = np.float32(1.0) / np.float32(float(d))          # IEEE division: RN_f32(1/d)
    assert Fraction(float(hi)) == Fraction(float(_rn32(1 / d)))
    assert lo == _rn32(1 / d - Fraction(float(hi)))


def test_two_operation_quotient_is_correctly_rounded_for_every_code():
    d, lo = _constants()
    hi = _rn32(1 / d)
    for y in range(-510, 511):
        fy = Fraction(y)
        low = _rn32(fy * Fraction(float(lo)))              # v_mul_f32
        got = _rn32(fy * Fraction(float(hi)) + Fraction(float(low)))   # fused multiply-add
        assert got == _rn32(fy / d), y


def test_single_product_is_not_enough():
    # The plain product y * RN(1/d) misrounds some codes, so the low part matters.
    d, _ = _constants()
    hi = _rn32(1 / d)
    bad = [y for y in range(-510, 511) if _rn32(Fraction(y) * Fraction(float(hi))) != _rn32(Fraction(y) / d)]
    assert len(bad) > 0
