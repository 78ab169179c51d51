"""Floating-point formats used by the codecs (oracle side).

bfloat16 values are carried as uint16 bit patterns; float16 uses numpy's
native type (its float32 -> float16 conversion rounds to nearest even).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    the rounded values as float64.  Used when a promoted window's content is
    rebuilt from its ledger (QEvict Algorithm 1: dequantize into the
    full-precision tier)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def fma32(a: np.ndarray, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    """float32(a*b + c) with a single rounding.

    a, b, c are float16 / small-integer values: the exact product and sum fit
    a float64 significand, so computing in float64 and rounding once is the
    fused multiply-add."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(np.float32)


FLT_MIN = float(np.finfo(np.float32).tiny)      # 2**-126
