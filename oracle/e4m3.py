"""E4M3 number format, table-based (oracle; test infrastructure only).

Source: "FP8 Mixed Precision: DeepSeek-V3 Training Architecture", section
"Why Naive FP8 Training Suffers Precision Collapse" gives E4M3 as 1 sign,
4 exponent and 3 mantissa bits with largest magnitude about 448, and section
"1. Fine-Grained Tile and Block-Wise Scaling" (equation for W_FP8) clips the
scaled values to [-448, 448].

Reading of the encoding (the pages give only the bit split and the maximum):
448 = 1.75 * 2**8 is reachable with 4 exponent bits only if the exponent bias
is 7 and the all-ones exponent still holds finite values, with only
S.1111.111 reserved for NaN and no infinities.  So:

* exponent field E = 0:  value = (-1)**S * (M / 8) * 2**-6     (subnormal)
* otherwise:             value = (-1)**S * (1 + M / 8) * 2**(E - 7)
* code 0x7F / 0xFF:      NaN

Encoding (saturating, round to nearest, ties to even):

1. NaN input -> 0x7F (a NaN produced by arithmetic has no defined sign, so
   the canonical positive NaN code is used).
2. a = min(|y|, 448): finite overflow and +-Inf saturate to 448.
3. a is compared exactly (in float64, where every grid value and every
   float32 input is exact) with the midpoints between adjacent non-negative
   grid values; the nearest grid value wins, an exact midpoint goes to the
   code with an even last bit.
4. The sign bit of y is ORed in, so negative values that round to zero give
   0x80.

This is deliberately a nearest-value search over a table, not bit
manipulation.
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def _build_tables():
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    grid = vals[:127].copy()          # non-negative finite values, codes 0..126
    assert np.all(np.diff(grid) > 0)
    mids = (grid[:-1] + grid[1:]) / 2.0   # exact in float64
    return vals, grid, mids


DECODE_TABLE, GRID, MIDPOINTS = _build_tables()


def decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values (exact); NaN for 0x7F/0xFF."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(y) -> np.ndarray:
    """Saturating round-to-nearest-even E4M3 encode of float32/float64 values.

    Inputs are taken at face value (float32 inputs are widened exactly).
    Returns uint8 codes with the shape of ``y``.
    """
    y = np.asarray(y)
    yf = y.astype(np.float64)
    nan = np.isnan(yf)
    a = np.minimum(np.abs(np.where(nan, 0.0, yf)), MAX_FINITE)
    idx = np.searchsorted(MIDPOINTS, a, side="left")      # first midpoint >= a
    idx_c = np.minimum(idx, len(MIDPOINTS) - 1)
    tie = (idx < len(MIDPOINTS)) & (a == MIDPOINTS[idx_c])
    # at a tie between grid[idx] and grid[idx + 1] pick the even code
    code = np.where(tie & (idx % 2 == 1), idx + 1, idx).astype(np.uint8)
    code = code | np.where(np.signbit(yf), 0x80, 0).astype(np.uint8)
    code = np.where(nan, NAN_CODE, code).astype(np.uint8)
    return code
