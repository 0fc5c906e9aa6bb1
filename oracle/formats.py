"""Codes of the two 4-bit weight formats and their scale bytes (FP64, exact).

Sources:
* EdgeRock-4B-NVFP4 model card, opening description: NVFP4 stores E2M1 codes,
  an E4M3 scale byte for each group of 16 weights, and a per-matrix FP32 factor.
  The E2M1 and E4M3 value sets are the OCP microscaling / OCP FP8 definitions
  those names refer to.
* ROCmFP4 design page, section 01 (values) and the
  format comparison table: the Codebook10 grid 0, +-1, +-2, +-3, +-4, +-6, +-8,
  +-10, E2M1-derived with the outer magnitude retuned from 12 to 10; scales
  are unsigned E4M3 (UE4M3) and the search scores the finite candidates.
* Same page, comparison table, stock Q4_0 column: a uniform integer grid, one
  FP16 scale per 32 weights.

Readings (the pages leave these open):
* Codebook10 code order: codes 0..6 are twice the E2M1 magnitude of the same
  code, code 7 is 10 (the retuned 12); bit 3 is the sign. Code 8 is level 0.
* UE4M3: the byte's bit 7 is ignored (masked); 0x7F is NaN and never emitted,
  so the finite candidates are the 127 codes 0x00..0x7E, zero included.
* Q4_0: the 16 codes are the consecutive integers -8..7 (code q is level q - 8),
  the usual stock Q4_0 grid: the comparison table's evenly spaced integers in 4 bits.
"""
from __future__ import annotations

import numpy as np

E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
CODEBOOK10_MAGNITUDE = np.array([0.0, 1.0, 2.0, 3.0, 4.0, 6.0, 8.0, 10.0], dtype=np.float64)

UE4M3_FINITE_CODES = 127  # 0x00 .. 0x7E


def e2m1_value(code) -> np.ndarray:
    """E2M1 nibble -> value. Bit 3 is the sign (code 8 is -0.0)."""
    c = np.asarray(code, dtype=np.int64)
    mag = E2M1_MAGNITUDE[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def codebook10_value(code) -> np.ndarray:
    """Codebook10 nibble -> integer level in {0, +-1, +-2, +-3, +-4, +-6, +-8, +-10}."""
    c = np.asarray(code, dtype=np.int64)
    mag = CODEBOOK10_MAGNITUDE[c & 7]
    return np.where(((c & 8) != 0) & (mag != 0.0), -mag, mag)


def q4_0_value(code) -> np.ndarray:
    """Q4_0 nibble -> integer level q - 8 in -8..7."""
    return np.asarray(code, dtype=np.int64).astype(np.float64) - 8.0


def fp16_value(bits) -> np.ndarray:
    """IEEE binary16 bit pattern (uint16) -> exact FP64 value."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def fp16_encode_rne(v) -> np.ndarray:
    """FP64 value -> IEEE binary16 bit pattern, round to nearest even (numpy's conversion)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def e4m3_value(byte) -> np.ndarray:
    """OCP FP8 E4M3 ("fn") byte -> value: bias 7, no infinities, S.1111.111 is NaN.

    normal:    (-1)^s * (8 + m) * 2^(e - 10)   for e in 1..15
    subnormal: (-1)^s * m * 2^-9               for e = 0
    """
    b = np.asarray(byte, dtype=np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2((e - 10).astype(np.float64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def ue4m3_value(byte) -> np.ndarray:
    """Unsigned E4M3 scale byte -> value (bit 7 masked off)."""
    return e4m3_value(np.asarray(byte, dtype=np.int64) & 0x7F)


# The 127 finite non-negative E4M3 values, in code order (strictly increasing).
E4M3_POSITIVE_GRID = e4m3_value(np.arange(UE4M3_FINITE_CODES))


def e4m3_encode_rne(v) -> np.ndarray:
    """Non-negative FP64 value -> nearest finite E4M3 code 0x00..0x7E.

    Ties go to the even code. Values above 448 saturate to 0x7E. Every midpoint
    between neighbouring grid values is exact in FP64, so the comparison is exact.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode_rne takes finite non-negative values")
    grid = E4M3_POSITIVE_GRID
    hi = np.clip(np.searchsorted(grid, v, side="left"), 1, UE4M3_FINITE_CODES - 1)
    lo = hi - 1
    mid = (grid[lo] + grid[hi]) * 0.5
    code = np.where(v < mid, lo, np.where(v > mid, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(v >= grid[-1], UE4M3_FINITE_CODES - 1, code)
    return code.astype(np.uint8)
