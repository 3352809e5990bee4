"""Exact rounding helpers for the oracle (test infrastructure only).

fp16 and fp32 rounding use numpy's IEEE casts (round to nearest, ties to
even).  The OCP 8-bit E4M3 format ("FN" variant: 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits, no infinities, one NaN pattern per sign, largest
finite value 448, smallest normal 2^-6, subnormal spacing 2^-9) is written out
here from that definition; it is the FP8 format that the "[FP8 3/4] Integrate
FP8 attention and caching into TabICLv2" page quantises Q/K/V to.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6
E4M3_MANT_BITS = 3
E4M3_BIAS = 7


def f32(x):
    """Round to IEEE binary32 (nearest even)."""
    return np.asarray(x).astype(np.float32)


def f16(x):
    """Round to IEEE binary16 (nearest even), directly from the input's precision."""
    return np.asarray(x).astype(np.float16)


def e4m3_round(x) -> np.ndarray:
    """Round finite values with |x| <= 448 to the nearest E4M3 value, ties to even.

    The binade of |x| is e = floor(log2|x|), but never below the smallest
    normal exponent -6 (below it the grid is the uniform subnormal grid);
    the grid spacing in that binade is 2^(e-3).  Returned as float64 values,
    which hold every E4M3 value exactly.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(~np.isfinite(a)) or np.any(a > E4M3_MAX):
        raise ValueError("e4m3_round expects finite inputs already clamped to +-448")
    _, E = np.frexp(a)                      # a = m * 2**E with m in [0.5, 1)
    e = np.maximum(E - 1, E4M3_MIN_NORMAL_EXP)
    spacing = np.ldexp(1.0, e - E4M3_MANT_BITS)
    r = np.round(a / spacing) * spacing     # np.round: half to even; the division is exact
    return np.copysign(r, x)


def e4m3_encode(v) -> np.ndarray:
    """Bit pattern (uint8) of values that lie on the E4M3 grid (|v| <= 448)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.signbit(v).astype(np.uint8) << 7
    sub = a < 2.0 ** E4M3_MIN_NORMAL_EXP
    _, E = np.frexp(np.where(sub, 1.0, a))
    e = E - 1
    exp_field = np.where(sub, 0, e + E4M3_BIAS)
    mant = np.where(sub, a / 2.0 ** (E4M3_MIN_NORMAL_EXP - E4M3_MANT_BITS),
                    (a / np.ldexp(1.0, e) - 1.0) * (1 << E4M3_MANT_BITS))
    if np.any(mant != np.floor(mant)):
        raise ValueError("e4m3_encode: value not on the E4M3 grid")
    return (sign | (exp_field.astype(np.uint8) << 3) | mant.astype(np.uint8)).astype(np.uint8)


def e4m3_decode_table() -> np.ndarray:
    """float64 value of every E4M3 bit pattern 0..255 (NaN for S.1111.111)."""
    codes = np.arange(256)
    sign = np.where(codes & 0x80, -1.0, 1.0)
    exp_field = (codes >> 3) & 0xF
    mant = codes & 0x7
    normal = sign * (1.0 + mant / 8.0) * np.ldexp(1.0, exp_field - E4M3_BIAS)
    subn = sign * mant * 2.0 ** (E4M3_MIN_NORMAL_EXP - E4M3_MANT_BITS)
    val = np.where(exp_field == 0, subn, normal)
    val[(codes & 0x7F) == 0x7F] = np.nan
    return val


E4M3_VALUES = e4m3_decode_table()
