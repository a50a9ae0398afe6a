"""Exact-rational helpers for pinning the oracle (CPU tests only).

These are written from the IEEE 754 definitions with Python Fractions and share
nothing with the oracle's C code: rounding a rational to binary32 / binary16
(round to nearest, ties to even) and rounding to an integer (ties to even).
"""
from fractions import Fraction

import numpy as np


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # adjust: 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def rne_int(a: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    f = a.numerator // a.denominator           # floor
    rem = a - f
    if rem > Fraction(1, 2):
        return f + 1
    if rem < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def _round_to_format(a: Fraction, man_bits: int, emin: int, emax: int) -> Fraction:
    """Nearest value of a binary format (man_bits explicit mantissa bits,
    normal exponents emin..emax, subnormals), ties to even; overflow -> inf (None)."""
    if a == 0:
        return Fraction(0)
    sign = -1 if a < 0 else 1
    a = abs(a)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - man_bits)
    r = rne_int(a / quantum)
    v = r * quantum
    max_finite = (2 - Fraction(2) ** (-man_bits)) * Fraction(2) ** emax
    if v > max_finite:
        return None
    return sign * v


def round_f32(a: Fraction):
    return _round_to_format(a, 23, -126, 127)


def round_f16(a: Fraction):
    return _round_to_format(a, 10, -14, 15)


def f16_value(bits: int) -> Fraction:
    """Exact value of binary16 bits (finite only), from the format definition."""
    s = -1 if (bits >> 15) & 1 else 1
    E = (bits >> 10) & 0x1F
    man = bits & 0x3FF
    assert E != 31
    if E == 0:
        return s * Fraction(man, 2 ** 24)
    return s * Fraction(1024 + man) * Fraction(2) ** (E - 25)


def f32_frac(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def quantize_block_exact(w, bits: int):
    """Quantize one block of 32 binary32 values by exact arithmetic.

    Returns (codes list, scale as Fraction). Mirrors the stated rule only:
    scale = binary16(binary32(amax / Q)); code = clamp(rne(binary32(w / scale))).
    """
    Q = {4: 7, 5: 15, 8: 127}[bits]
    lo, hi = -Q - 1, Q
    ws = [f32_frac(v) for v in w]
    amax = max(abs(v) for v in ws)
    s32 = round_f32(amax / Q)
    s16 = round_f16(s32)
    if s16 == 0:
        return [0] * len(ws), Fraction(0)
    codes = []
    for v in ws:
        r = round_f32(v / s16)
        codes.append(min(hi, max(lo, rne_int(r))))
    return codes, s16


def signed5(t: int) -> int:
    """The unique v in [-16, 15] congruent to t modulo 32."""
    return [v for v in range(-16, 16) if (v - t) % 32 == 0][0]


def signed_nibble(t: int) -> int:
    """The unique v in [-8, 7] congruent to t modulo 16."""
    return [v for v in range(-8, 8) if (v - t) % 16 == 0][0]
