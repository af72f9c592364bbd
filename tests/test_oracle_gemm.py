"""Pins for the oracle's block-scaled GEMM and its output rounding (CPU only).

Pinned by: exact rational brute force on tiny shapes (asymmetric scales, so a
transposed scale table or a dropped block fails), the lossless fixture where
the result must equal the plain float64 matmul of the BF16 inputs, the
unit-scale fixture (a plain FP8 GEMM), the one-block closed form, cross-layout
identities, and an independent BF16 rounding reference.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, gemm, quant
import synthetic as syn


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)   # no NaN codes


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (2, 3, 256), (4, 4, 384), (3, 2, 128)])
def test_brute_force_fractions(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A, B = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    KB = K // 128
    sA = (rng.random((M, KB)) * 3 + 0.01).astype(np.float32)
    sB = (rng.random((N, KB)) * 3 + 0.01).astype(np.float32)
    R = gemm.block_gemm(A, sA, B, sB)
    for i in range(M):
        for j in range(N):
            tot = Fraction(0)
            for kb in range(KB):
                part = sum(Fraction(float(e4m3.decode(A[i, k]))) * Fraction(float(e4m3.decode(B[j, k])))
                           for k in range(kb * 128, kb * 128 + 128))
                tot += Fraction(float(sA[i, kb])) * Fraction(float(sB[j, kb])) * part
            assert abs(Fraction(R[i, j]) - tot) <= abs(tot) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_block_partials_exact_any_order():
    rng = np.random.default_rng(1)
    A, B = _rand_codes(rng, (8, 128)), _rand_codes(rng, (8, 128))
    a, b = e4m3.decode(A), e4m3.decode(B)
    blas = a @ b.T
    naive = np.zeros((8, 8))
    for k in range(127, -1, -1):                 # reversed sequential order
        naive += a[:, k:k + 1] * b[:, k][None, :]
    assert np.array_equal(blas, naive)


def test_lossless_fixture_equals_plain_matmul():
    xb, _ = syn.lossless_tiles(64, 384, seed=2, tile=(1, 128), k_range=(-4, 4))
    wb, _ = syn.lossless_tiles(256, 384, seed=3, tile=(128, 128), k_range=(-4, 4))
    Xq, sX = quant.quant_rows(xb)
    Wq, sW = quant.quant_weight(wb)
    R = gemm.fprop(Xq, sX, Wq, sW)
    X = quant.bf16_to_f32(xb).astype(np.float64)
    W = quant.bf16_to_f32(wb).astype(np.float64)
    ref = X @ W.T
    assert np.allclose(R, ref, rtol=1e-14, atol=0)


def test_unit_scale_fixture_plain_fp8_gemm():
    rng = np.random.default_rng(4)
    A, B = _rand_codes(rng, (16, 256)), _rand_codes(rng, (32, 256))
    ones_a, ones_b = np.ones((16, 2), np.float32), np.ones((32, 2), np.float32)
    R = gemm.block_gemm(A, ones_a, B, ones_b)
    assert np.array_equal(R, e4m3.decode(A) @ e4m3.decode(B).T)


def test_one_block_closed_form_toy_layer():
    xb, wb = syn.toy_layer(0)
    Xq, sX = quant.quant_rows(xb)
    Wq, sW = quant.quant_weight(wb)
    R = gemm.fprop(Xq, sX, Wq, sW)
    closed = sX.astype(np.float64) * sW[:, 0].repeat(128)[None, :].astype(np.float64) \
        * (e4m3.decode(Xq) @ e4m3.decode(Wq).T)
    assert np.allclose(R, closed, rtol=1e-15, atol=0)
    # the outlier tile (row 0) has its own scale 20/448; other rows do not
    assert sX[0, 0] == np.float32(np.float32(20.0) / np.float32(448))
    assert np.all(sX[1:, 0] < sX[0, 0])


def test_dgrad_equals_fprop_on_transposed_weights():
    rng = np.random.default_rng(5)
    dyb = syn.gaussian((32, 384), seed=6, std=1e-3)
    wb = syn.gaussian((384, 256), seed=7, std=0.02)      # W stored [d_out][d_in]
    dYq, s_dY = quant.quant_rows(dyb)
    Wq, sW = quant.quant_weight(wb)
    a, T = gemm.dgrad(dYq, s_dY, Wq, sW, with_magnitude=True)
    b = gemm.fprop(dYq, s_dY, np.ascontiguousarray(Wq.T), np.ascontiguousarray(sW.T))
    assert np.array_equal(a, b)
    # against the dense dequantized product (dequantize-then-matmul is equal in exact arithmetic)
    ref = quant.dequant_rows(dYq, s_dY) @ quant.dequant_weight(Wq, sW)
    assert np.all(np.abs(a - ref) <= 1e-13 * T)
    del rng


def test_wgrad_matches_dense_dequantized():
    dyb = syn.gaussian((256, 384), seed=8, std=1e-3)    # [tokens][d_out]
    xb = syn.activation_with_outliers(256, 128, seed=9)  # [tokens][d_in]
    dYt, s_dy = quant.quant_cols(dyb)
    Xt, s_x = quant.quant_cols(xb)
    R, T = gemm.wgrad(dYt, s_dy, Xt, s_x, with_magnitude=True)
    ref = quant.dequant_rows(dYt, s_dy) @ quant.dequant_rows(Xt, s_x).T
    assert R.shape == (384, 128)
    assert np.all(np.abs(R - ref) <= 1e-13 * T)


def test_grouped_equals_per_expert():
    counts = np.array([3, 0, 130, 1])
    off = syn.expert_offsets(counts)
    xb = syn.activation_with_outliers(int(counts.sum()), 256, seed=10)
    Xq, sX = quant.quant_rows(xb)
    Wq_e, sW_e = zip(*[quant.quant_weight(syn.gaussian((128, 256), seed=20 + e, std=0.02))
                       for e in range(4)])
    R = gemm.grouped_fprop(Xq, sX, off, Wq_e, sW_e)
    for e in range(4):
        lo, hi = off[e], off[e + 1]
        assert np.array_equal(R[lo:hi], gemm.fprop(Xq[lo:hi], sX[lo:hi], Wq_e[e], sW_e[e]))


def _bf16_rne_from_f32(x32):
    b = x32.view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def test_round_to_bf16_against_integer_rne():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 32, size=500_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    x = x[np.abs(x) < np.float32(3.3e38)]
    assert np.array_equal(gemm.round_to_bf16_bits(x.astype(np.float64)), _bf16_rne_from_f32(x))


def test_round_to_bf16_no_double_rounding():
    # 1 + 2**-8 + 2**-40 is just above a BF16 midpoint; a detour through fp32
    # would land exactly on the midpoint and round down to 1.0
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert gemm.round_to_bf16_bits(np.array([v]))[0] == 0x3F81
    assert gemm.round_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80   # tie -> even
    assert gemm.round_to_bf16_bits(np.array([-(2.0 ** -134)]))[0] == 0x8000     # tie -> -0
    assert gemm.round_to_bf16_bits(np.array([3 * 2.0 ** -134]))[0] == 0x0002
    assert gemm.round_to_bf16_bits(np.array([3.4e38]))[0] == 0x7F80
    assert gemm.round_to_bf16_bits(np.array([np.nan]))[0] == 0x7FC0


def test_round_to_bf16_special_values_match_torch():
    # torch's CPU float32 -> bfloat16 cast (round to nearest even) on values
    # where one rounding from float64 and one from float32 agree
    import torch
    v = np.array([np.inf, -np.inf, 0.0, -0.0, 1.0, -3.0, 2.0 ** -133, -(2.0 ** -126),
                  3.3895e38, -3.3895e38, 3.4e38, 65504.0, 1e-40], np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gemm.round_to_bf16_bits(v.astype(np.float64)), want)


def test_ulp_bf16():
    assert gemm.ulp_bf16(np.array([1.0]))[0] == 2.0 ** -7
    assert gemm.ulp_bf16(np.array([1.99]))[0] == 2.0 ** -7
    assert gemm.ulp_bf16(np.array([-2.0]))[0] == 2.0 ** -6
    assert gemm.ulp_bf16(np.array([0.0]))[0] == 2.0 ** -133
