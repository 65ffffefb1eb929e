"""Exact rational arithmetic used to pin the oracle on small inputs.

Independent of the oracle: values are Python Fractions, rounding to a
binary format is done here from the format's definition (p significant bits,
a least exponent, ties to the even significand), and E4M3 encoding is a
brute-force search over every finite code's value.
"""
from fractions import Fraction
import math
import struct


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_f32(u):
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def round_to_format(q, p, emin, emax=None):
    """Round the exact rational q to the nearest number with p significant
    bits and exponent >= emin (subnormals below), ties to even significand.
    Returns a Fraction, or +-inf (float) on overflow beyond emax."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix e so that 2^e <= a < 2^(e+1) exactly
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (p - 1))
    m = a / quantum
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * quantum
    if emax is not None and r >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * r


def round_f32(q):
    """Exact binary32 round-to-nearest-even of a rational; returns a float."""
    r = round_to_format(q, 24, -126, 127)
    if isinstance(r, float):
        return r
    return float(r)


def add_f32(a, b):
    return round_f32(Fraction(a) + Fraction(b))


def mul_f32(a, b):
    return round_f32(Fraction(a) * Fraction(b))


def div_f32(a, b):
    return round_f32(Fraction(a) / Fraction(b))


def bf16_round(x):
    """Nearest bf16 value of a finite float x (8 significant bits), as float."""
    r = round_to_format(Fraction(x), 8, -126, 127)
    return r if isinstance(r, float) else float(r)


def e4m3_value(code):
    """Value of an OCP E4M3 code from the format definition (None for NaN)."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    f = code & 7
    if e == 15 and f == 7:
        return None
    if e == 0:
        return s * Fraction(f, 512)
    return s * (1 + Fraction(f, 8)) * Fraction(2) ** (e - 7)


E4M3_FINITE = [(c, e4m3_value(c)) for c in range(0x7F)]  # magnitudes 0..0x7E


def e4m3_nearest(v, negative):
    """Brute force: the finite E4M3 magnitude nearest |v|, ties to the even
    code, anything at or above 448 saturating to 448."""
    sign = 0x80 if negative else 0
    if isinstance(v, float) and math.isnan(v):
        return 0x7F | sign
    if isinstance(v, float) and math.isinf(v):
        return 0x7E | sign
    m = abs(Fraction(v))
    if m >= 448:
        return 0x7E | sign
    best = None
    for c, val in E4M3_FINITE:
        d = abs(val - m)
        if best is None or d < best[1] or (d == best[1] and c % 2 == 0):
            best = (c, d)
    return best[0] | sign
