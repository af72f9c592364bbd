"""Tile size and percentile clipping of the activation scales (oracle; test
infrastructure only).

Sources:

* "Fine-Grained FP8 Quantization in DeepSeek", section 2 (one scale per tile
  of contiguous values; smaller tiles keep an outlier's damage local) and its
  study lab (tiled max scaling, error against tile size, the cost of the
  scale metadata).
* "Online Quantization During Training", section 4 (percentile clipping
  trades clipping of the largest values for resolution of the rest) and its
  failure-modes list (clipping can erase rare but important values).

Readings taken where the pages leave a step open:

* A tile is 1 x T contiguous values of a row, T in {32, 64, 128, 256, 512,
  1024}, anchored at column 0 (cols % T == 0); the scale layout is the
  row quantizer's, one FP32 scale per tile.
* Percentile clipping clips at an order statistic of the tile's magnitudes:
  with rank r, the clip value c is the r-th largest |x| (r = 1: the max, the
  online rule), s = max(fl32(c / 448), fl32(1e-12)), and the r - 1 values
  above c saturate.  For a tile of T values this is the (1 - (r-1)/T)
  quantile taken without interpolation.
* A tile containing NaN keeps the online rule's convention (NaN scale,
  every code NaN), whatever the rank.
"""
from __future__ import annotations

import numpy as np

from . import quant

TILES = (32, 64, 128, 256, 512, 1024)


def tile_scales(x_bits, tile: int, rank: int = 1) -> np.ndarray:
    """s[rows][cols/tile] from the rank-th largest |x| of each tile."""
    x = quant.bf16_to_f32(x_bits)
    M, K = x.shape
    assert K % tile == 0 and 1 <= rank <= tile
    g = np.abs(x.reshape(M, K // tile, tile))
    has_nan = np.isnan(g).any(-1)
    srt = -np.sort(-np.where(np.isnan(g), np.float32(0), g), axis=-1)   # descending
    c = srt[..., rank - 1].astype(np.float32)
    s = quant.scale_from_amax(c)
    return np.where(has_nan, quant.CANONICAL_NAN, s).astype(np.float32)


def quant_rows_tiles(x_bits, tile: int, rank: int = 1):
    """Codes [rows][cols], scales [rows][cols/tile] and the saturation count."""
    x = quant.bf16_to_f32(x_bits)
    M, K = x.shape
    s = tile_scales(x_bits, tile, rank)
    q, _, _, sat = quant._quantize_groups(x.reshape(M, K // tile, tile), s)
    return q.reshape(M, K), s, sat


def dequant_tiles(q, s, tile: int) -> np.ndarray:
    """float64 reconstruction decode(q) * s, exact."""
    from . import e4m3
    return e4m3.decode(q) * np.repeat(np.asarray(s, np.float64), tile, axis=1)


def metadata_bytes_per_value(tile: int) -> float:
    """FP32 scale bytes per quantized value: 4 / T (0.03125 at T = 128)."""
    return 4.0 / tile
