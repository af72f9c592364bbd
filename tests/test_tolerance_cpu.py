"""The GEMM tolerance helper itself (host logic, no GPU): the truncation
bound evaluated at chosen positions equals the full bound there, and
check_gemm puts elements in the right class and rejects what it must."""
import numpy as np
import pytest

from oracle import gemm as og
from oracle import quant
import synthetic as syn
from tolerance import RECORDS, check_gemm, truncation_bound, truncation_bound_at


def small_problem(M=40, N=256, K=384):
    Xq, sX = quant.quant_rows(syn.activation_with_outliers(M, K, seed=201))
    Wq, sW = quant.quant_weight(syn.gaussian((N, K), seed=202, std=0.02))
    return Xq, sX, Wq, og.expand_block_scales(sW, N), sW


def test_truncation_bound_at_equals_the_full_bound():
    Xq, sX, Wq, sWn, _ = small_problem()
    E = truncation_bound(Xq, sX, Wq, sWn)
    rng = np.random.default_rng(3)
    r = rng.integers(0, Xq.shape[0], 500)
    c = rng.integers(0, Wq.shape[0], 500)
    got = truncation_bound_at(Xq, sX, Wq, sWn, r, c, chunk=128)
    assert np.array_equal(got, E[r, c])


def test_exact_result_is_all_within_2ulp():
    Xq, sX, Wq, sWn, sW = small_problem()
    R, T = og.fprop(Xq, sX, Wq, sW, with_magnitude=True)
    y = og.round_to_bf16_bits(R)
    st = check_gemm(y, R, T, Xq.shape[1], label="exact")
    assert st["within_2ulp"] == st["n"] == R.size
    assert st["exact_match"] == R.size
    assert st["fp32_sum_bound"] == st["truncation_bound"] == st["failed"] == 0
    assert RECORDS[-1]["label"] == "exact"


def test_classes_and_a_planted_error():
    n = 100000          # enough elements that two large errors stay below 1e-3 normwise
    R = np.linspace(1.0, 2.0, n).reshape(1000, 100)
    T = np.full_like(R, 1.0)
    E = np.zeros_like(R)
    yv = R.copy()
    # element (0, 0): cancellation (T >> |R|), error beyond 2 ulp (0.0156),
    # within the plain FP32-summation bound (~0.082)
    T[0, 0] = 1e4
    yv[0, 0] = R[0, 0] + 0.05
    # element (0, 1): beyond the plain bound, within the truncation bound (~0.52)
    T[0, 1] = 1e4
    E[0, 1] = 0.5
    yv[0, 1] = R[0, 1] + 0.3
    y = og.round_to_bf16_bits(yv)
    st = check_gemm(y, R, T, 128, E=E, label="classes")
    assert st["within_2ulp"] == n - 2
    assert st["fp32_sum_bound"] == 1 and st["truncation_bound"] == 1 and st["failed"] == 0
    # the same through E_at (only the two elements beyond 2 ulp are asked for)
    asked = []

    def E_at(r, c):
        asked.append((tuple(r), tuple(c)))
        return E[r, c]

    st2 = check_gemm(y, R, T, 128, E_at=E_at, label="classes E_at")
    assert asked == [((0, 0), (0, 1))]
    assert (st2["fp32_sum_bound"], st2["truncation_bound"]) == (1, 1)
    # a planted error: 4 ulp off where nothing cancels
    y_bad = og.round_to_bf16_bits(R.copy())
    y_bad[1, 7] = og.round_to_bf16_bits(np.array([R[1, 7] * (1 + 4 * 2.0 ** -7)]))[0]
    with pytest.raises(AssertionError, match="outside both bounds"):
        check_gemm(y_bad, R, T, 128, E=np.zeros_like(R), label="planted")
    assert RECORDS[-1]["failed"] == 1


def test_nan_pattern_must_match():
    R = np.ones((2, 4))
    R[1, 2] = np.nan
    T = np.ones_like(R)
    y = og.round_to_bf16_bits(np.ones_like(R))
    with pytest.raises(AssertionError, match="NaN pattern"):
        check_gemm(y, R, T, 128, E=np.zeros_like(R))
