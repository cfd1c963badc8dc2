"""Exact decoding of fp16 and bf16 bit patterns (oracle; test infrastructure).

Written from the IEEE-754 field definitions, not from a conversion routine:

  binary16: sign 1 bit, exponent 5 bits (bias 15), fraction 10 bits.
    e = 0      -> (-1)^s * f * 2^-24            (zero / subnormal)
    0 < e < 31 -> (-1)^s * (1024 + f) * 2^(e-25)
    e = 31     -> inf (f = 0) or NaN
  bfloat16: sign 1, exponent 8 (bias 127), fraction 7 (the top half of f32).
    e = 0      -> (-1)^s * f * 2^-133
    0 < e < 255-> (-1)^s * (128 + f) * 2^(e-134)
    e = 255    -> inf / NaN

Every such value is exact in float64 and in float32.  Subnormals are kept:
block scales drawn as 1e-3*|N(0,1)| are fp16-subnormal about 5% of the time.
"""
from __future__ import annotations

import numpy as np


def _decode(bits: np.ndarray, ebits: int, fbits: int) -> np.ndarray:
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    emax = (1 << ebits) - 1
    bias = emax >> 1
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> fbits) & emax
    f = (b & ((1 << fbits) - 1)).astype(np.float64)
    implicit = float(1 << fbits)
    # normal: (2^fbits + f) * 2^(e - bias - fbits); subnormal: f * 2^(1 - bias - fbits)
    normal = np.ldexp(implicit + f, (e - bias - fbits).astype(np.int64))
    sub = np.ldexp(f, 1 - bias - fbits)
    val = np.where(e == 0, sub, normal)
    special = np.where(f == 0, np.inf, np.nan)
    val = np.where(e == emax, special, val)
    return sign * val


def f16_to_f64(bits) -> np.ndarray:
    """fp16 bit patterns -> exact float64 values."""
    return _decode(bits, 5, 10)


def f16_to_f32(bits) -> np.ndarray:
    """fp16 bit patterns -> float32 (exact: every binary16 value is a binary32 value)."""
    return f16_to_f64(bits).astype(np.float32)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    return _decode(bits, 8, 7)


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return bf16_to_f64(bits).astype(np.float32)
