"""OCP E4M3FN codec in float64 (oracle; test infrastructure only).

Format [paper.rainbus.top summary, 前置知识 "FP8 块级混合精度训练": 4 exponent
bits and 3 mantissa bits]. The variant with a 448 maximum, no infinities and a
single NaN mantissa pattern (OCP "FN") is the reading taken here, because the
blocks are scaled so that their maximum lands at or below 448.

Bit layout: s eeee mmm, bias 7.
  e == 0        : value = (m / 8) * 2^-6      (subnormals, quantum 2^-9)
  1 <= e <= 15  : value = (1 + m / 8) * 2^(e - 7), except e == 15, m == 7 (NaN)
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6
_SUB_QUANTUM_INV = 2.0 ** 9


def e4m3_table() -> np.ndarray:
    """float64[256]: decoded value of every code (NaN for 0x7F and 0xFF)."""
    codes = np.arange(256, dtype=np.int64)
    s = codes >> 7
    e = (codes >> 3) & 0xF
    m = codes & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    val[(codes & 0x7F) == 0x7F] = np.nan
    return val


_TABLE = e4m3_table()


def decode_e4m3(q: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (exact)."""
    return _TABLE[np.asarray(q, dtype=np.uint8)]


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """float64 values with |v| <= 448 -> uint8 codes, round to nearest, ties to even.

    The sign bit is kept for results that round to zero (-0 and tiny negative
    values give 0x80).
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("encode_e4m3: non-finite input")
    a = np.abs(v)
    if a.size and a.max() > E4M3_MAX:
        raise ValueError("encode_e4m3: |v| > 448 is outside the block-scaled range")
    # subnormal range: integer number of 2^-9 quanta, half to even; 8 quanta is the
    # smallest normal 2^-6 whose code 0x08 continues the same integer sequence
    q_sub = np.rint(a * _SUB_QUANTUM_INV).astype(np.int64)
    # normal range: a = f * 2^x with f in [0.5, 1): exponent x - 1, significand 2f in [1, 2)
    f, x = np.frexp(np.where(a >= _MIN_NORMAL, a, 1.0))
    exp = x.astype(np.int64) - 1
    frac8 = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)  # 0..8, half to even
    carry = frac8 == 8
    exp = np.where(carry, exp + 1, exp)
    frac8 = np.where(carry, 0, frac8)
    q_norm = ((exp + 7) << 3) | frac8
    code = np.where(a < _MIN_NORMAL, q_sub, q_norm)
    code = code | (np.signbit(v).astype(np.int64) << 7)
    return code.astype(np.uint8)
