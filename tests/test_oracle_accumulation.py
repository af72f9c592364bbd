"""Pins for the oracle's accumulation models (CPU only).

Pinned by: the limited-precision running sum at 24 bits with rounding to
nearest-even equals float32 accumulation done by numpy one addition at a
time (a library routine), and at 53 bits equals float64 accumulation; the
exact sum against exact rational arithmetic on a tiny case; the promoted
sum with one interval covering all of K equals the exact sum rounded once to
FP32, and with interval 1 equals float32 accumulation of the products;
closed-form cases of the pages' "small terms fall off" picture (a 14-bit sum
keeps 1 + 2**-13, a 13-bit one loses it).
"""
from fractions import Fraction

import numpy as np

from oracle import accumulation as acc
from oracle import e4m3


def _codes(shape, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(shape).astype(np.float32) * np.float32(30)
    return e4m3.encode(v)


def test_exact_against_fractions():
    A, B = _codes((3, 256), 1), _codes((4, 256), 2)
    R = acc.exact(A, B)
    a, b = e4m3.decode(A), e4m3.decode(B)
    for m in range(3):
        for n in range(4):
            want = sum(Fraction(float(a[m, k])) * Fraction(float(b[n, k])) for k in range(256))
            assert Fraction(R[m, n]) == want


def test_running_sum_24_bits_is_float32_accumulation():
    A, B = _codes((5, 384), 3), _codes((6, 384), 4)
    got = acc.running_sum(A, B, 24, "rne")
    a = e4m3.decode(A).astype(np.float32)
    b = e4m3.decode(B).astype(np.float32)
    s = np.zeros((5, 6), np.float32)
    for k in range(384):
        s = s + np.outer(a[:, k], b[:, k]).astype(np.float32)   # products exact in float32
    assert np.array_equal(got, s.astype(np.float64))


def test_running_sum_53_bits_is_float64_accumulation():
    A, B = _codes((4, 256), 5), _codes((4, 256), 6)
    a, b = e4m3.decode(A), e4m3.decode(B)
    s = np.zeros((4, 4))
    for k in range(256):
        s = s + np.outer(a[:, k], b[:, k])
    assert np.array_equal(acc.running_sum(A, B, 53), s)
    assert np.array_equal(s, acc.exact(A, B))          # exact at this size


def test_running_sum_small_terms_fall_off():
    one = int(e4m3.encode(np.float32(1.0)))
    tiny13 = int(e4m3.encode(np.float32(2.0 ** -6)))   # 2**-6 * 2**-7 = 2**-13 below
    A = np.array([[one, tiny13, tiny13]], np.uint8)
    B = np.array([[one, int(e4m3.encode(np.float32(2.0 ** -7))), 0]], np.uint8)
    # 1 + 2**-13 needs 14 significant bits: kept at 14, lost at 13 (trunc)
    assert acc.running_sum(A, B, 14, "trunc")[0, 0] == 1.0 + 2.0 ** -13
    assert acc.running_sum(A, B, 13, "trunc")[0, 0] == 1.0
    assert acc.running_sum(A, B, 13, "rne")[0, 0] == 1.0     # tie -> even


def test_promoted_limits():
    A, B = _codes((4, 512), 7), _codes((5, 512), 8)
    R = acc.exact(A, B)
    assert np.array_equal(acc.promoted(A, B, 512), R.astype(np.float32).astype(np.float64))
    assert np.array_equal(acc.promoted(A, B, 1), acc.running_sum(A, B, 24, "rne"))


def test_relative_errors_closed_form():
    R = np.array([[1.0, -2.0], [4.0, 0.0]])
    C = np.array([[1.5, -2.0], [4.0, 1.0]])
    e = acc.relative_errors(C, R, T=np.full((2, 2), 10.0))
    assert np.isclose(e["norm"], np.sqrt(0.25 + 1.0) / np.sqrt(21.0))
    assert e["median_rel"] == 0.0 and np.isclose(e["max_over_T"], 0.1)


def test_fourteen_bit_picture_matches_the_pages_figure():
    # "Introduction to LLM Quantization" section 3: with about 14 bits of
    # accumulation, K = 4096 gives relative errors of up to about 2%.  The
    # running-sum model at 14 bits (nearest-even) on Gaussian FP8 products:
    # the tail of the per-element relative error sits at that figure.
    A, B = _codes((32, 4096), 11), _codes((32, 4096), 12)
    e = acc.relative_errors(acc.running_sum(A, B, 14, "rne"), acc.exact(A, B))
    assert 0.005 < e["p99_rel"] < 0.1
    assert e["norm"] < 0.005                 # the bulk stays well below it
    e24 = acc.relative_errors(acc.running_sum(A, B, 24, "rne"), acc.exact(A, B))
    assert e24["p99_rel"] < 1e-4             # FP32 accumulation: no such tail
