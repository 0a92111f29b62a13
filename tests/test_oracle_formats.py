"""Pins for the oracle's number formats (CPU only).

Each of the 256 E4M3 codes and 256 E8M0 codes is checked against the format
definition, re-derived here with exact rationals from the bit fields (a second,
independent reading of the OCP E4M3FN and E8M0 definitions; it shares no code
with the oracle).  bf16 rounding is checked against exact rational
round-half-even.
"""
import math
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle


def e4m3_exact(code):
    """OCP E4M3FN: s.eeee.mmm, bias 7, subnormals 0.mmm*2^-6, S.1111.111 NaN."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return None  # NaN
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 2 ** 6)
    return s * (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


def test_e4m3_all_codes():
    nan_codes = []
    for c in range(256):
        ref = e4m3_exact(c)
        got = oracle.e4m3(c)
        if ref is None:
            assert math.isnan(got)
            nan_codes.append(c)
        else:
            assert Fraction(got) == ref, (c, got, ref)
    assert nan_codes == [0x7F, 0xFF]


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x30, 0.5), (0x40, 2.0), (0xB8, -1.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
    (0x08, 2.0 ** -6), (0x7E, 448.0), (0xFE, -448.0), (0x00, 0.0), (0x3C, 1.5), (0x78, 256.0)])
def test_e4m3_spot_values(code, value):
    assert oracle.e4m3(code) == value


def test_e4m3_negative_zero():
    v = oracle.e4m3(0x80)
    assert v == 0.0 and math.copysign(1.0, v) == -1.0


def test_e8m0_all_codes():
    for c in range(255):
        assert Fraction(oracle.e8m0(c)) == Fraction(2) ** (c - 127), c
    assert math.isnan(oracle.e8m0(0xFF))
    assert oracle.e8m0(0x7F) == 1.0
    assert oracle.e8m0(0x00) == 2.0 ** -127
    assert oracle.e8m0(0xFE) == 2.0 ** 127


def bf16_rne_exact(x):
    """Exact rational round-half-even of a finite float to bfloat16 bits."""
    if x == 0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    sign = 0x8000 if x < 0 else 0
    a = Fraction(abs(x))
    # exponent: floor(log2 a)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = max(e, -126) - 7  # spacing exponent
    scaled = a / Fraction(2) ** q
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = Fraction(fl) * Fraction(2) ** q
    if v >= Fraction(2) ** 128:
        return sign | 0x7F80
    if v < Fraction(2) ** -126:
        return sign | int(v / Fraction(2) ** -133)
    e2 = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e2 > v:
        e2 -= 1
    mant = int((v / Fraction(2) ** e2 - 1) * 128)
    return sign | ((e2 + 127) << 7) | mant


def test_bf16_rne_against_exact_rounding():
    rng = random.Random(7)
    vals = [1.0, -1.0, 64.0, 40.0, -32.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -40,
            2.0 ** -126, 2.0 ** -130, 2.0 ** -133, 3 * 2.0 ** -134, 2.0 ** -134, (2 - 2 ** -8) * 2.0 ** 127,
            (2 - 2 ** -9) * 2.0 ** 127, 1e30, -1e-30, 0.1, 1 / 3]
    for _ in range(3000):
        vals.append(rng.uniform(-1, 1) * 2.0 ** rng.randint(-140, 127))
    for _ in range(500):  # exact ties between bf16 neighbours
        m = rng.randint(128, 255)
        vals.append((m + 0.5) * 2.0 ** rng.randint(-120, 100))
    got = oracle.to_bf16_bits(np.array(vals))
    for v, g in zip(vals, got):
        assert int(g) == bf16_rne_exact(v), (v, hex(int(g)), hex(bf16_rne_exact(v)))


def test_bf16_special():
    got = oracle.to_bf16_bits(np.array([np.nan, np.inf, -np.inf, 0.0, -0.0]))
    assert [hex(int(x)) for x in got] == ["0x7fc0", "0x7f80", "0xff80", "0x0", "0x8000"]
