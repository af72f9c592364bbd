"""Pins for the oracle's tile-size and percentile-clipping quantizer (CPU).

Pinned by: T = 128 with rank 1 is the row quantizer (itself pinned); for
every tile size, lossless tiles come back exactly with scales 2**k known in
closed form; a tile built by hand gives the clip value, scale, codes and
saturation count of each rank; NaN and Inf tiles follow the online rule's
convention; the mean error falls with the tile size on the outlier recipe
(the pages' reason for small tiles); the metadata cost is 4 / T bytes.
"""
import numpy as np
import pytest

from oracle import e4m3, granularity as gr, quant
import synthetic as syn


def test_tile_128_rank_1_is_the_row_quantizer():
    x = syn.activation_with_outliers(64, 1024, seed=3)
    q, s, sat = gr.quant_rows_tiles(x, 128, 1)
    q0, s0 = quant.quant_rows(x)
    assert np.array_equal(q, q0) and np.array_equal(s.view(np.uint32), s0.view(np.uint32))
    assert sat == 0


@pytest.mark.parametrize("tile", gr.TILES)
def test_lossless_tiles_every_size(tile):
    bits, k = syn.lossless_tiles(24, 2048, seed=tile, tile=(1, tile))
    q, s, sat = gr.quant_rows_tiles(bits, tile, 1)
    assert np.array_equal(s, np.exp2(k).astype(np.float32))
    assert np.array_equal(gr.dequant_tiles(q, s, tile), quant.bf16_to_f32(bits).astype(np.float64))
    assert sat == 0


def test_rank_by_hand():
    row = np.zeros(128, np.float32)
    row[:4] = [1000.0, -896.0, 800.0, 5.0]
    row[4:] = 1.0
    x = syn.f32_to_bf16_bits(row[None, :])
    for rank, c, n_sat in ((1, 1000.0, 0), (2, 896.0, 1), (3, 800.0, 2), (4, 5.0, 3), (5, 1.0, 4)):
        q, s, sat = gr.quant_rows_tiles(x, 128, rank)
        assert s[0, 0] == np.float32(np.float32(c) / np.float32(448)), rank
        assert sat == n_sat, rank
        assert q[0, rank - 1] in (0x7E, 0xFE)                     # the clip value maps to +-448
        assert np.all(q[0, :rank - 1] & 0x7F == 0x7E)             # the values above it saturate
    # rank 2 on 896 / (896/448): exactly 448 -> code 0xFE (negative)
    q, s, _ = gr.quant_rows_tiles(x, 128, 2)
    assert q[0, 1] == 0xFE and e4m3.decode(np.uint8(q[0, 0])) == 448.0


def test_ties_do_not_saturate():
    row = np.full(64, 0.5, np.float32)
    row[:3] = 7.0
    q, s, sat = gr.quant_rows_tiles(syn.f32_to_bf16_bits(row[None, :]), 64, 3)
    assert s[0, 0] == np.float32(7.0 / 448) and sat == 0


def test_nan_and_inf_tiles():
    row = np.ones(256, np.float32)
    row[3] = np.nan
    row[130] = np.inf
    row[131] = 2.0
    x = syn.f32_to_bf16_bits(row[None, :])
    q, s, sat = gr.quant_rows_tiles(x, 128, 2)
    assert s.view(np.uint32)[0, 0] == 0x7FC00000 and np.all(q[0, :128] == 0x7F)
    assert s[0, 1] == np.float32(2.0 / 448)                       # rank 2 skips the Inf
    assert q[0, 130] == 0x7E and sat == 1                         # Inf saturates to 448
    q1, s1, _ = gr.quant_rows_tiles(x, 128, 1)
    assert s1[0, 1] == np.inf                                     # online rule: scale Inf


def test_error_falls_with_tile_size():
    x = syn.activation_with_outliers(128, 4096, seed=5)
    xf = quant.bf16_to_f32(x).astype(np.float64)
    err = {}
    for tile in gr.TILES:
        q, s, _ = gr.quant_rows_tiles(x, tile, 1)
        err[tile] = np.mean(np.abs(gr.dequant_tiles(q, s, tile) - xf)) / np.mean(np.abs(xf))
    vals = [err[t] for t in gr.TILES]
    assert all(a < b for a, b in zip(vals, vals[1:])), err


def test_metadata_bytes():
    assert gr.metadata_bytes_per_value(128) == 0.03125
    assert [gr.metadata_bytes_per_value(t) * t for t in gr.TILES] == [4.0] * 6
