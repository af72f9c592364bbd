"""Pins for the oracle's fine-grained quantizers (CPU only).

Pinned by: a lossless fixture whose scales and codes are known in closed
form (catches tile orientation, anchoring, and scale formula mistakes), the
tile-max -> 448 invariant, idempotence, the E4M3 error bound, special tiles,
an exact-rational brute force on tiny inputs, and an independent PyTorch CPU
implementation of the same rule.
"""
from fractions import Fraction

import numpy as np
import torch

from oracle import e4m3, quant
import synthetic as syn


def test_scale_floor_bits():
    assert quant.SCALE_FLOOR.view(np.uint32) == 0x2B8CBCCC


def test_lossless_rows_known_scales_and_codes():
    bits, k = syn.lossless_tiles(64, 1024, seed=3, tile=(1, 128))
    q, s = quant.quant_rows(bits)
    assert np.array_equal(s, np.exp2(k).astype(np.float32))        # s = 2**k exactly
    x = quant.bf16_to_f32(bits).astype(np.float64)
    assert np.array_equal(quant.dequant_rows(q, s), x)             # exact reconstruction
    # codes equal the direct encode of x / 2**k
    v = x / np.repeat(np.exp2(k), 128, axis=1)
    assert np.array_equal(q, e4m3.encode(v))


def test_lossless_weight_blocks_known_scales():
    bits, k = syn.lossless_tiles(384, 256, seed=4, tile=(128, 128))
    q, s = quant.quant_weight(bits)
    assert s.shape == (3, 2)
    assert np.array_equal(s, np.exp2(k).astype(np.float32))
    assert np.array_equal(quant.dequant_weight(q, s), quant.bf16_to_f32(bits).astype(np.float64))


def test_lossless_cols_known_scales():
    bits, k = syn.lossless_tiles(256, 96, seed=5, tile=(128, 1))
    qt, s = quant.quant_cols(bits)
    assert qt.shape == (96, 256) and s.shape == (96, 2)
    assert np.array_equal(s, np.exp2(k).T.astype(np.float32))
    x_t = quant.bf16_to_f32(bits).T.astype(np.float64)
    assert np.array_equal(quant.dequant_rows(qt, s), x_t)


def test_orientation_matters():
    # row tiles of a lossless-by-column input are NOT lossless: catches swapped axes
    bits, _ = syn.lossless_tiles(256, 256, seed=6, tile=(128, 1))
    q, s = quant.quant_rows(bits)
    assert not np.array_equal(quant.dequant_rows(q, s), quant.bf16_to_f32(bits).astype(np.float64))


def _random_tiles(seed=0):
    bits = syn.activation_with_outliers(96, 1024, seed=seed)
    extra = syn.gaussian((32, 1024), seed=seed + 1, std=1e-30)     # tiny values: floor path
    return np.concatenate([bits, extra])


def test_tile_max_encodes_to_448_and_sign():
    bits = _random_tiles()
    x = quant.bf16_to_f32(bits)
    q, s = quant.quant_rows(bits)
    M, K = x.shape
    xt = np.abs(x.reshape(M, K // 128, 128))
    qt = q.reshape(M, K // 128, 128)
    arg = np.argmax(xt, axis=-1)
    qmax = np.take_along_axis(qt, arg[..., None], -1)[..., 0]
    amax = xt.max(-1)
    big = amax >= np.float32(448e-12)
    assert np.all((qmax[big] & 0x7F) == 0x7E)
    # floor applies to tiny tiles: no code reaches 448 there
    assert np.all(s[~big] == quant.SCALE_FLOOR) and np.all((qmax[~big] & 0x7F) < 0x7E)
    nz = x != 0
    assert np.all(((q >> 7) == 1)[nz] == np.signbit(x)[nz])


def test_idempotent_requantization():
    bits = _random_tiles(7)
    q, s = quant.quant_rows(bits)
    M, K = q.shape
    deq32 = (e4m3.decode(q).reshape(M, K // 128, 128) * s[..., None].astype(np.float64)).astype(np.float32)
    again = e4m3.encode((deq32 / s[..., None]).astype(np.float32)).reshape(M, K)
    assert np.array_equal(again, q)


def test_error_bound_e4m3():
    bits = _random_tiles(8)
    x = quant.bf16_to_f32(bits).astype(np.float64)
    q, s = quant.quant_rows(bits)
    deq = quant.dequant_rows(q, s)
    sfull = np.repeat(s.astype(np.float64), 128, axis=1)
    normal = np.abs(x / sfull) >= 2.0 ** -6
    err = np.abs(x - deq)
    slack = 1 + 2.0 ** -19
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * slack)
    assert np.all(err[~normal] <= 2.0 ** -10 * sfull[~normal] * slack)


def test_monotone_within_tile():
    bits = _random_tiles(9)
    x = quant.bf16_to_f32(bits)
    q, _ = quant.quant_rows(bits)
    for r in range(0, x.shape[0], 17):
        for t in range(0, x.shape[1], 128):
            xs, qs = x[r, t:t + 128], q[r, t:t + 128]
            o = np.argsort(xs, kind="stable")
            assert np.all(np.diff(e4m3.decode(qs[o])) >= 0)


def test_special_tiles():
    def bf(vals):
        return syn.f32_to_bf16_bits(np.asarray(vals, np.float32)).reshape(1, 128)

    zero = np.zeros(128, np.float32); zero[::2] = -0.0
    q, s = quant.quant_rows(bf(zero))
    assert s[0, 0] == quant.SCALE_FLOOR
    assert np.array_equal(q[0], np.where(np.signbit(zero), 0x80, 0x00))

    nan = np.ones(128, np.float32); nan[5] = np.nan
    q, s = quant.quant_rows(bf(nan))
    assert s.view(np.uint32)[0, 0] == 0x7FC00000 and np.all(q == 0x7F)

    inf = np.linspace(-3, 3, 128).astype(np.float32); inf[7] = -np.inf
    q, s = quant.quant_rows(bf(inf))
    assert np.isposinf(s[0, 0])
    fin = np.arange(128) != 7
    assert q[0, 7] == 0x7F
    assert np.all((q[0][fin] & 0x7F) == 0)
    assert np.array_equal(q[0][fin] >> 7, np.signbit(inf[fin]).astype(np.uint8))

    sub = np.zeros(128, np.float32); sub[3] = 2.0 ** -130; sub[9] = -(2.0 ** -133)
    q, s = quant.quant_rows(bf(sub))
    assert s[0, 0] == quant.SCALE_FLOOR       # BF16 subnormal tile: floor scale
    assert q[0, 9] == 0x80 and q[0, 3] == 0x00


def test_brute_force_rational_tiny():
    # exact rational arithmetic for s and x/s on a few tiles, then nearest code
    rng = np.random.default_rng(11)
    bits = syn.f32_to_bf16_bits((rng.standard_normal((3, 256)) * 3).astype(np.float32))
    q, s = quant.quant_rows(bits)
    x = quant.bf16_to_f32(bits)
    grid = [Fraction(float(g)) for g in e4m3.GRID]
    for r in range(3):
        for t in range(2):
            tile = x[r, 128 * t:128 * (t + 1)]
            amax = max(abs(Fraction(float(v))) for v in tile)
            s_exact = np.float32(float(amax / 448))              # fl32 of the exact ratio
            s_exact = max(s_exact, np.float32(1e-12))
            assert s[r, t] == s_exact
            for i, v in enumerate(tile):
                y = np.float32(float(Fraction(float(v)) / Fraction(float(s_exact))))
                a = min(abs(Fraction(float(y))), Fraction(448))
                d = [abs(a - g) for g in grid]
                c = [j for j, dj in enumerate(d) if dj == min(d)]
                code = c[0] if len(c) == 1 else [j for j in c if j % 2 == 0][0]
                code |= 0x80 if np.signbit(y) else 0
                assert q[r, 128 * t + i] == code


def test_against_torch_cpu_implementation():
    bits = _random_tiles(12)
    x = torch.from_numpy(quant.bf16_to_f32(bits)).reshape(128, 8, 128)
    amax = x.abs().amax(-1)
    s = torch.clamp(amax / 448.0, min=float(np.float32(1e-12)))
    q = (x / s[..., None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    q_o, s_o = quant.quant_rows(bits)
    assert np.array_equal(s.numpy(), s_o)
    assert np.array_equal(q.reshape(128, 1024).numpy(), q_o)


def test_weight_blocks_match_rowwise_definition():
    # each 128x128 block uses one amax over all 16384 values
    bits = syn.gaussian((256, 384), seed=13, std=0.02)
    q, s = quant.quant_weight(bits)
    w = quant.bf16_to_f32(bits)
    for i in range(2):
        for j in range(3):
            blk = w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
            assert s[i, j] == np.float32(np.abs(blk).max() / np.float32(448))
            qe = e4m3.encode((blk / s[i, j]).astype(np.float32))
            assert np.array_equal(q[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)], qe)


def test_external_scales_and_saturation_count():
    bits = syn.gaussian((4, 256), seed=14)
    x = quant.bf16_to_f32(bits)
    s = np.full((4, 2), np.float32(0.001))
    q, amax, sat = quant.quant_rows_external(bits, s)
    y = (x / np.float32(0.001)).astype(np.float32)
    assert sat == int(np.count_nonzero(np.abs(y) > 464))
    assert sat > 0 and np.all((q[np.abs(y) > 448] & 0x7F) == 0x7E)
    # a value that only rounds down onto 448 is not counted as clipped
    edge = syn.f32_to_bf16_bits(np.array([0.46, 0.464, 0.4641, -0.5] + [0.0] * 124, np.float32))
    _, _, sat_e = quant.quant_rows_external(edge.reshape(1, 128), np.full((1, 1), np.float32(0.001)))
    ye = (quant.bf16_to_f32(edge) / np.float32(0.001)).astype(np.float32)
    assert sat_e == int(np.count_nonzero(np.abs(ye) > 464)) and sat_e >= 1
    assert np.array_equal(amax, np.abs(x).reshape(4, 2, 128).max(-1))
    # online scales passed back in reproduce the online codes and never saturate
    q_on, s_on = quant.quant_rows(bits)
    q2, _, sat2 = quant.quant_rows_external(bits, s_on)
    assert np.array_equal(q2, q_on) and sat2 == 0
