"""Operand-tiled byte layout of E4M3 weight codes (oracle; test infrastructure
only).

Source: "Fine-Grained FP8 Quantization in DeepSeek", section 4 and its
failure-modes list: the kernels load FP8 values with their local scales, and
the layout of operands and scale metadata decides real performance.  The
layout below is this library's GEMM-ready form of a code matrix; the oracle
defines it from its formula, element by element.

For codes Q [R][C] (R % 16 == 0, C % 128 == 0) the tiled array T has R * C
bytes.  Element (r, c) sits at

    ((r // 16) * (C // 128) + c // 128) * 2048      16-row x 128-column tile
  + ((c % 128) // 64) * 1024                        which 64-column half
  + (((c % 64) // 16) * 16 + r % 16) * 16           lane slot: 16-column group, row
  + c % 16                                          byte in the slot

so one 1 KB half-tile is what 64 lanes load as 16 bytes each, lane
16 g + i getting row i, columns 64 h + 16 g .. + 16.
"""
from __future__ import annotations

import numpy as np


def tiled_offset(r, c, C: int):
    r = np.asarray(r, np.int64)
    c = np.asarray(c, np.int64)
    return (((r // 16) * (C // 128) + c // 128) * 2048 + ((c % 128) // 64) * 1024
            + (((c % 64) // 16) * 16 + r % 16) * 16 + c % 16)


def tile_codes(q) -> np.ndarray:
    """Row-major codes [R][C] -> the tiled byte array (R * C,)."""
    q = np.asarray(q, np.uint8)
    R, C = q.shape
    assert R % 16 == 0 and C % 128 == 0
    out = np.zeros(R * C, np.uint8)
    r, c = np.meshgrid(np.arange(R), np.arange(C), indexing="ij")
    out[tiled_offset(r, c, C)] = q
    return out


def untile_codes(t, R: int, C: int) -> np.ndarray:
    t = np.asarray(t, np.uint8).reshape(-1)
    r, c = np.meshgrid(np.arange(R), np.arange(C), indexing="ij")
    return t[tiled_offset(r, c, C)]
