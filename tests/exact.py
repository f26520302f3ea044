"""Exact rational reference arithmetic for pinning the oracle (test helper, independent of it).

Everything here works on ``fractions.Fraction`` values, so it is exact by construction and shares
no code or floating-point arithmetic with ``oracle/``.
"""

from __future__ import annotations

import struct
from fractions import Fraction


def f32_to_fraction(x: float) -> Fraction:
    """Exact value of a float32 (given as a Python float that is float32-representable)."""
    return Fraction(struct.unpack("<f", struct.pack("<f", x))[0])


def f32_bits_to_fraction(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0])


def bf16_bits_to_fraction(bits: int) -> Fraction:
    return f32_bits_to_fraction((bits & 0xFFFF) << 16)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_to_binary(fr: Fraction, sig_bits: int, emin: int, emax: int | None = None) -> Fraction:
    """Round ``fr`` to nearest, ties to even, in a binary format with ``sig_bits`` significant bits
    and smallest normal exponent ``emin`` (gradual underflow below it). Returns an exact Fraction,
    or +-inf as a float when the magnitude overflows past ``emax``."""
    if fr == 0:
        return Fraction(0)
    neg = fr < 0
    a = -fr if neg else fr
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (sig_bits - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if emax is not None and r >= Fraction(2) ** (emax + 1):
        return float("-inf") if neg else float("inf")
    return -r if neg else r


def round_to_f32(fr: Fraction) -> Fraction:
    return round_to_binary(fr, 24, -126, 127)


def round_to_bf16(fr: Fraction) -> Fraction:
    return round_to_binary(fr, 8, -126, 127)
