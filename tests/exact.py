"""Exact rational arithmetic for checking the oracle: IEEE rounding of a rational number to a
binary format with p significant bits, done with ``fractions.Fraction`` and no floating point.

This is a second, independent route to the same definitions the oracle implements in C with
binary32/binary64 arithmetic, so a slip in either shows up as a disagreement.
"""
import decimal
import struct
from fractions import Fraction

BF16_P, BF16_EMIN = 8, -126      # bf16: 8 significant bits, binary32's exponent range
F32_P, F32_EMIN = 24, -126       # binary32
BF16_MAX = Fraction(2) ** 128 - Fraction(2) ** 120  # (2 - 2^-7) * 2^127


def floor_log2(a):
    """The integer e with 2^e <= a < 2^(e+1), for a rational a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_nearest_even(q, p, emin):
    """q rounded to the nearest number with p significant bits (spacing fixed below 2^emin),
    ties to the even neighbour. Returns a Fraction; no overflow handling."""
    q = Fraction(q)
    if q == 0:
        return q
    sign = -1 if q < 0 else 1
    a = abs(q)
    qe = max(floor_log2(a), emin) - (p - 1)     # exponent of the spacing at a
    step = Fraction(2) ** qe
    units = a / step
    lower = units.numerator // units.denominator
    rem = units - lower
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lower % 2 == 1):
        lower += 1
    return sign * lower * step


def f32(q):
    return round_nearest_even(q, F32_P, F32_EMIN)


def bf16_value(q):
    """The bf16 value nearest to q (a Fraction), or +-inf (as a float) past the largest finite."""
    r = round_nearest_even(q, BF16_P, BF16_EMIN)
    if abs(r) > BF16_MAX:
        return float("inf") if r > 0 else float("-inf")
    return r


def bits_of_value(v, negative_zero=False):
    """Raw bf16 bits of a value that is exactly representable in bf16 (Fraction, int or float)."""
    if v == 0:
        return 0x8000 if negative_zero else 0x0000
    f = float(v)
    (u,) = struct.unpack("<I", struct.pack("<f", f))
    if u & 0xFFFF:
        raise ValueError(f"{v} is not a bf16 value")
    return u >> 16


def value_of_bits(b):
    """The exact value (Fraction) of finite bf16 bits."""
    (f,) = struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))
    return Fraction(f)


def bf16_bits(q):
    """Bits of the correctly rounded bf16 of a rational q (q != -0)."""
    r = bf16_value(q)
    if isinstance(r, float):
        return 0x7F80 if r > 0 else 0xFF80
    if r == 0:
        return 0x8000 if q < 0 else 0x0000
    return bits_of_value(r)


def sqrt_fraction(q, digits=60):
    """sqrt(q) to ``digits`` significant decimal digits, as a Fraction."""
    ctx = decimal.Context(prec=digits)
    d = ctx.divide(decimal.Decimal(q.numerator), decimal.Decimal(q.denominator))
    return Fraction(ctx.sqrt(d))


def near_bf16_tie(y, rel=Fraction(1, 10**12)):
    """True if y lies within a relative distance ``rel`` of a bf16 rounding tie point."""
    if y == 0:
        return False
    a = abs(y)
    qe = max(floor_log2(a), BF16_EMIN) - (BF16_P - 1)
    step = Fraction(2) ** qe
    units = a / step
    frac = units - (units.numerator // units.denominator)
    return abs(frac - Fraction(1, 2)) * step <= rel * a
