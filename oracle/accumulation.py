"""Accumulation precision of FP8 GEMMs (oracle; test infrastructure only).

Sources:

* "Introduction to LLM Quantization", section 3 (increasing accumulation
  precision): Hopper tensor cores keep GEMM sums with about 14 bits, far
  below FP32, and with a large inner dimension (K = 4096) the page puts the
  resulting relative error at up to about 2%; DeepSeek's answer is to move
  partial sums into FP32 at a fixed interval.
* "FP8 Mixed Precision: DeepSeek-V3 Training Architecture", section 3
  (decoupled accumulation): partial products go into FP32 registers.
* "Making Low Precision Work", Idea 3 (accumulate in high precision):
  small terms added to a growing running total in low precision are lost.

What is modelled here:

* ``exact`` - the sum of the FP8 products, exact (float64 block partials,
  see ``oracle.gemm``): the reference every scheme is measured against.
* ``running_sum`` - the pages' picture of a limited-precision accumulator:
  the products (exact) are added one at a time in k order and the running
  sum is kept to ``bits`` significant bits after every addition, rounded to
  nearest-even or truncated toward zero.  The pages give the width (about
  14 bits) but not the rounding; both are offered.
* ``promoted`` - the method's decoupling with an ideal matrix unit: the
  products of each ``interval`` consecutive k are summed exactly, the partial
  is rounded once to FP32 and added to an FP32 running sum (round to
  nearest-even): what per-interval promotion costs on its own.
"""
from __future__ import annotations

import numpy as np

from . import e4m3


def _products(Aq, Bq) -> np.ndarray:
    """P[m, n, k] = A[m, k] * B[n, k] exactly (float64)."""
    A = e4m3.decode(np.asarray(Aq, np.uint8))
    B = e4m3.decode(np.asarray(Bq, np.uint8))
    return A[:, None, :] * B[None, :, :]


def exact(Aq, Bq) -> np.ndarray:
    """C[m, n] = sum_k A[m, k] B[n, k], exact: every partial of E4M3 products
    is a multiple of 2**-18 below 2**53 * 2**-18 here (K <= 2**17)."""
    A = e4m3.decode(np.asarray(Aq, np.uint8))
    B = e4m3.decode(np.asarray(Bq, np.uint8))
    K = A.shape[1]
    assert K <= 1 << 17
    C = np.zeros((A.shape[0], B.shape[0]))
    for k0 in range(0, K, 128):            # exact block partials, exact sum of them
        C += A[:, k0:k0 + 128] @ B[:, k0:k0 + 128].T
    return C


def round_sig(x, bits: int, mode: str = "rne") -> np.ndarray:
    """x rounded to ``bits`` significant bits (no exponent limits)."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                     # x = m 2**e, 0.5 <= |m| < 1
    scaled = np.ldexp(m, bits)
    r = np.rint(scaled) if mode == "rne" else np.trunc(scaled)
    return np.ldexp(r, e - bits)


def running_sum(Aq, Bq, bits: int, mode: str = "rne") -> np.ndarray:
    """Products added in k order into a sum kept to ``bits`` significant bits."""
    P = _products(Aq, Bq)
    s = np.zeros(P.shape[:2])
    for k in range(P.shape[2]):
        s = round_sig(s + P[:, :, k], bits, mode)   # s + p is exact in float64 here
    return s


def promoted(Aq, Bq, interval: int) -> np.ndarray:
    """Each run of ``interval`` k summed exactly and rounded once to FP32, the
    rounded partials added in order into an FP32 running sum (RNE)."""
    A = e4m3.decode(np.asarray(Aq, np.uint8))
    B = e4m3.decode(np.asarray(Bq, np.uint8))
    K = A.shape[1]
    acc = np.zeros((A.shape[0], B.shape[0]), np.float32)
    for k0 in range(0, K, interval):
        part = np.zeros(acc.shape)
        for j0 in range(k0, min(K, k0 + interval), 128):       # exact partial
            j1 = min(K, k0 + interval, j0 + 128)
            part += A[:, j0:j1] @ B[:, j0:j1].T
        # the sum of two FP32 values is exact in float64 or so lopsided that
        # rounding it to float64 first cannot change its FP32 rounding
        acc = (acc.astype(np.float64) + part.astype(np.float32).astype(np.float64)).astype(np.float32)
    return acc.astype(np.float64)


def relative_errors(C, R, T=None) -> dict:
    """Normwise ||C - R|| / ||R||, the median and 99th percentile of
    |C - R| / |R| over elements with R != 0, and (with T = sum |a b|)
    max |C - R| / T."""
    C = np.asarray(C, np.float64)
    R = np.asarray(R, np.float64)
    d = np.abs(C - R)
    nz = R != 0
    out = {"norm": float(np.linalg.norm(C - R) / np.linalg.norm(R)),
           "median_rel": float(np.median(d[nz] / np.abs(R[nz]))),
           "p99_rel": float(np.quantile(d[nz] / np.abs(R[nz]), 0.99))}
    if T is not None:
        out["max_over_T"] = float(np.max(d / np.asarray(T, np.float64)))
    return out
