"""FP8 E4M3 codec, written out from the format's definition. TEST INFRASTRUCTURE (oracle).

Format (FP8-RL write-up, section 1: 4 exponent bits, 3 mantissa bits, range [-448, 448]; the
Unified-FP8 blog's "FP8 data format" section names the OCP FP8 white paper as the definition):
an 8-bit code c has sign s = bit 7, biased exponent E = bits 6..3 (bias 7) and mantissa m = bits
2..0.

* E = 15 and m = 7 is NaN (codes 0x7F and 0xFF); there is no infinity;
* E = 0 is subnormal: value (-1)^s * m * 2^-9 (m = 0 gives a signed zero);
* otherwise the value is (-1)^s * (1 + m / 8) * 2^(E - 7).

The largest finite magnitude is code 0x7E = 1.75 * 2^8 = 448, matching the stated range.

``encode`` rounds a float32 to the nearest code, ties to the even mantissa, and saturates
magnitudes above 448 to +-448. It works on the integer bit pattern of the float32, so it involves
no floating-point arithmetic at all.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODES = (0x7F, 0xFF)


def decode(codes) -> np.ndarray:
    """Value of each E4M3 code as float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 255)):
        raise ValueError("E4M3 codes are bytes")
    s = c >> 7
    E = (c >> 3) & 15
    m = c & 7
    subnormal = np.ldexp(m.astype(np.float64), -9)
    normal = np.ldexp((8 + m).astype(np.float64), (E - 10).astype(np.int64))
    mag = np.where(E == 0, subnormal, normal)
    val = np.where(s == 1, -mag, mag)
    return np.where((E == 15) & (m == 7), np.nan, val)


def _round_shift_half_even(x: np.ndarray, sh) -> np.ndarray:
    """round(x / 2^sh) with ties to even, for integers 0 <= x < 2^24 and shifts 1 <= sh <= 30."""
    x = x.astype(np.uint32)
    sh = np.asarray(sh).astype(np.uint32)
    q = x >> sh
    rem = x - (q << sh)
    half = np.left_shift(np.uint32(1), sh - np.uint32(1))
    up = (rem > half) | ((rem == half) & ((q & np.uint32(1)) == np.uint32(1)))
    return q + up.astype(np.uint32)


def encode(values) -> np.ndarray:
    """Nearest E4M3 code (ties to even, saturating at +-448) of each float32 value.

    The sign bit is always carried over, so -0.0 and negative values that round to zero give 0x80.
    NaN gives 0x7F with the sign kept; +-inf saturates like any magnitude above 448.
    """
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    bits = v.view(np.uint32)
    sign = (bits >> np.uint32(31)) << np.uint32(7)
    a = bits & np.uint32(0x7FFFFFFF)
    exp = (a >> np.uint32(23)).astype(np.int32)
    frac = a & np.uint32(0x7FFFFF)

    # |v| >= 2^-6: E4M3 normal range. Keep 3 of the 23 fraction bits, round the other 20.
    e = exp - 127
    q = _round_shift_half_even(frac, 20).astype(np.int32)
    carry = q == 8  # rounding overflowed the 3-bit mantissa: next binade
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    normal_code = ((e + 7) << 3) | q

    # |v| < 2^-6: E4M3 subnormal range, a grid of step 2^-9. |v| * 2^9 = mant * 2^(e2 - 141),
    # with mant the 24-bit significand (no hidden bit for float32 subnormals).
    is_sub32 = exp == 0
    mant = np.where(is_sub32, frac, frac | np.uint32(0x800000))
    e2 = np.where(is_sub32, 1, exp)
    sh = np.clip(141 - e2, 1, 30)  # shifts >= 25 already round every mant < 2^24 to 0
    sub_code = _round_shift_half_even(mant, sh).astype(np.int32)  # 0..8

    small = a < np.uint32(0x3C800000)  # 2^-6
    code = np.where(small, sub_code, normal_code)
    too_big = (a > np.uint32(0x43E00000)) | (~small & ((e > 8) | ((e == 8) & (q > 6))))
    code = np.where(too_big, 0x7E, code)
    code = np.where(a > np.uint32(0x7F800000), 0x7F, code)  # NaN
    return (code.astype(np.uint32) | sign).astype(np.uint8)


def finite_codes() -> np.ndarray:
    """All 254 codes that are not NaN."""
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]
