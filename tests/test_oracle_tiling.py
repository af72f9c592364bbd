"""Pins for the operand-tiled code layout (CPU only): offsets worked out by
hand from the layout's description, the layout is a permutation (every byte
lands once), round trip, and one 1 KB half-tile holds exactly the 16 rows x
64 columns a wave's 64 lanes load."""
import numpy as np

from oracle import tiling


def test_hand_offsets():
    C = 256                                        # two 128-column blocks
    assert tiling.tiled_offset(0, 0, C) == 0
    assert tiling.tiled_offset(1, 0, C) == 16      # next row: next lane slot
    assert tiling.tiled_offset(0, 15, C) == 15
    assert tiling.tiled_offset(0, 16, C) == 256    # next 16-column group: 16 lanes on
    assert tiling.tiled_offset(0, 64, C) == 1024   # second half of the tile
    assert tiling.tiled_offset(0, 128, C) == 2048  # next K block
    assert tiling.tiled_offset(16, 0, C) == 4096   # next row group (2 K blocks later)
    assert tiling.tiled_offset(17, 70, C) == 4096 + 1024 + (0 * 16 + 1) * 16 + 6


def test_permutation_and_round_trip():
    rng = np.random.default_rng(0)
    q = rng.integers(0, 256, (48, 384), dtype=np.uint8)
    r, c = np.meshgrid(np.arange(48), np.arange(384), indexing="ij")
    off = tiling.tiled_offset(r, c, 384)
    assert np.array_equal(np.sort(off.ravel()), np.arange(48 * 384))
    t = tiling.tile_codes(q)
    assert np.array_equal(tiling.untile_codes(t, 48, 384), q)


def test_half_tile_is_a_wave_load():
    q = np.arange(32 * 256, dtype=np.int64).reshape(32, 256)
    R, C = q.shape
    codes = (q % 251).astype(np.uint8)
    t = tiling.tile_codes(codes)
    # half-tile (row group 1, K block 1, half 1): lane 16 g + i, bytes 16 g..
    base = (1 * 2 + 1) * 2048 + 1024
    for lane in range(64):
        g, i = lane // 16, lane % 16
        want = codes[16 + i, 128 + 64 + 16 * g:128 + 64 + 16 * g + 16]
        assert np.array_equal(t[base + 16 * lane:base + 16 * lane + 16], want)
