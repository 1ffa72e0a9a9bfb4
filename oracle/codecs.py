"""bf16 and OCP FP8 E4M3 codecs for the oracle (test infrastructure only).

Both encoders work the same plain way: list every finite non-negative value of
the format in increasing order (decoded from its bit layout), find the two
neighbours of |v|, compare |v| with their exact midpoint (computed in fp64,
where every midpoint of these narrow formats is exact), and on a tie take the
neighbour whose code is even (its last mantissa bit is 0). The sign is applied
afterwards, so -0.0 and tiny negative values keep their sign bit.

Formats:
  * bf16: 1 sign, 8 exponent (bias 127), 7 mantissa bits; the upper half of an
    IEEE binary32. Overflow follows IEEE round-to-nearest-even: |v| at or above
    the midpoint between the largest finite value and 2^128 becomes infinity.
  * OCP FP8 E4M3 ("e4m3fn", OCP 8-bit Floating Point Specification, OFP8):
    1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0 holds
    subnormals m * 2^-9; S.1111.111 is NaN; there are no infinities; the
    largest finite magnitude is 0.1111.110 = 448. The encoder saturates:
    magnitudes at or above 448 (infinity included) encode as +-448.
"""
from __future__ import annotations

import numpy as np

__all__ = ["e4m3_decode", "e4m3_encode", "bf16_decode", "bf16_encode",
           "E4M3_MAX"]

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 7) & 1
    expo = (c >> 3) & 0xF
    mant = c & 0x7
    normal = np.ldexp((8 + mant).astype(np.float64), (expo - 10).astype(np.int64))
    subnormal = np.ldexp(mant.astype(np.float64), -9)
    mag = np.where(expo == 0, subnormal, normal)
    mag = np.where((expo == 15) & (mant == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact)."""
    b = np.asarray(bits).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def _nearest_even(a: np.ndarray, values: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Code of the table value nearest to a (a >= 0, float64), ties to even code.

    ``values`` is strictly increasing; inputs above the last value take the
    last code.
    """
    n = values.shape[0]
    i = np.searchsorted(values, a, side="right")       # values[i-1] <= a < values[i]
    lo = np.clip(i - 1, 0, n - 1)
    hi = np.clip(i, 0, n - 1)
    mid = (values[lo] + values[hi]) * 0.5                # exact for these formats
    take_hi = (a > mid) | ((a == mid) & ((codes[hi] & 1) == 0))
    return np.where(take_hi, codes[hi], codes[lo])


# Finite non-negative E4M3 codes are 0x00..0x7E; their values increase with the code.
_E4M3_CODES = np.arange(0x7F, dtype=np.int64)
_E4M3_VALUES = e4m3_decode(_E4M3_CODES)


def e4m3_encode(v) -> np.ndarray:
    """float32/float64 values -> E4M3 codes (uint8), nearest-even, saturating."""
    with np.errstate(invalid="ignore"):        # signalling NaN inputs stay NaN
        v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    code = _nearest_even(a, _E4M3_VALUES, _E4M3_CODES)
    code = np.where(nan, 0x7F, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


# Finite non-negative bf16 codes are 0x0000..0x7F7F; 0x7F80 (+inf) is appended
# with the value 2^128 so that overflow rounds as IEEE prescribes (the largest
# finite code 0x7F7F is odd, so a tie at the overflow midpoint goes to inf).
_BF16_CODES = np.arange(0x7F81, dtype=np.int64)
_BF16_VALUES = bf16_decode(_BF16_CODES[:-1]).astype(np.float64)
_BF16_VALUES = np.concatenate([_BF16_VALUES, [2.0 ** 128]])


def bf16_encode(v) -> np.ndarray:
    """float32/float64 values -> bf16 bit patterns (uint16), nearest-even.

    Rounds the given value once (an fp64 input is not first rounded to fp32).
    NaN becomes the quiet NaN 0x7FC0 with the input's sign.
    """
    with np.errstate(invalid="ignore"):        # signalling NaN inputs stay NaN
        v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    code = _nearest_even(a, _BF16_VALUES, _BF16_CODES)
    code = np.where(nan, 0x7FC0, code)
    return (code | np.where(neg, 0x8000, 0)).astype(np.uint16)
