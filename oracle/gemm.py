"""Block-scaled FP8 GEMM in float64 (oracle; test infrastructure only).

Sources:

* "FP8 Mixed Precision: DeepSeek-V3 Training Architecture", section 3
  ("Decoupled Accumulation in Tensor Core GEMMs"): E4M3 x E4M3 products,
  partial sums held in FP32, and the block scale product s_A * s_B multiplied
  into the accumulated sum rather than into the operands.
* "Fine-Grained FP8 Quantization in DeepSeek", section 4: kernels load FP8 values
  and their local scales, multiply in hardware and accumulate in a wider
  type.
* "Introduction to LLM Quantization", section 2 (fine-grained steps 1-4: one
  scale per block, block products on the matrix unit, the product rescaled
  by the blocks' scaling factors) and section 1 (y = W x computed with FP32
  accumulation and stored as BF16; input gradient from the output gradient
  and the weights; weight gradient from the input and the output gradient).

Reading of the printed GEMM equation, which puts the k-dependent scales
outside the sum over k: the scales are constant only within one 128-wide K
block, so the result is

    C[i, j] = sum_kb  sA[i, kb] * sB[j, kb] * sum_{k in kb} A[i, k] * B[j, k]

with A, B the decoded E4M3 operands (both stored K-contiguous here).

Exactness of the block partials: every E4M3 value is an integer multiple of
2**-9 with magnitude <= 448, so each product is a multiple of 2**-18 with
magnitude < 2**17.62 and any partial sum of at most 128 of them is an integer
below 2**42.62 in units of 2**-18.  Every such partial, in any summation
order, is exact in binary64, so a float64 BLAS matmul per K block returns the
exact block sums.  The only roundings left in the oracle are the float64
scale multiply and the sum over blocks (about 1e-16 relative); the result is
then rounded once to the output type.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

TILE = 128


def block_gemm(Aq, sA, Bq, sB, with_magnitude: bool = False):
    """R[i, j] = sum_kb sA[i, kb] * sB[j, kb] * (A_kb @ B_kb^T)[i, j] in float64.

    Aq: uint8 [M][K]; Bq: uint8 [N][K]; sA: float32 [M][K/128];
    sB: float32 [N][K/128] (one scale per output column and K block).
    With ``with_magnitude`` also returns
    T = sum_kb |sA sB| * (|A_kb| @ |B_kb|^T), the conditioning magnitude.
    """
    Aq = np.asarray(Aq, np.uint8)
    Bq = np.asarray(Bq, np.uint8)
    M, K = Aq.shape
    N, K2 = Bq.shape
    assert K == K2 and K % TILE == 0
    KB = K // TILE
    sA = np.asarray(sA, np.float32).astype(np.float64)
    sB = np.asarray(sB, np.float32).astype(np.float64)
    assert sA.shape == (M, KB) and sB.shape == (N, KB)
    A = e4m3.decode(Aq)
    B = e4m3.decode(Bq)
    R = np.zeros((M, N), dtype=np.float64)
    T = np.zeros((M, N), dtype=np.float64) if with_magnitude else None
    for kb in range(KB):
        sl = slice(kb * TILE, (kb + 1) * TILE)
        P = A[:, sl] @ B[:, sl].T                      # exact block partial
        scale = sA[:, kb:kb + 1] * sB[:, kb][None, :]  # exact product of two fp32
        R += scale * P
        if with_magnitude:
            T += np.abs(scale) * (np.abs(A[:, sl]) @ np.abs(B[:, sl]).T)
    return (R, T) if with_magnitude else R


def expand_block_scales(s_blocks, rows: int) -> np.ndarray:
    """[rows/128][KB] block scales -> [rows][KB] (one per row)."""
    return np.repeat(np.asarray(s_blocks, np.float32), TILE, axis=0)[:rows]


def fprop(Xq, sX, Wq, sW, with_magnitude=False):
    """Y = X W^T: X_q [M][K] with 1x128 scales sX [M][K/128];
    W_q [N][K] with 128x128 block scales sW [N/128][K/128]."""
    N = np.asarray(Wq).shape[0]
    return block_gemm(Xq, sX, Wq, expand_block_scales(sW, N), with_magnitude)


def dgrad(dYq, s_dY, Wq, sW, with_magnitude=False):
    """dX = dY W: dY_q [M][Nout] with 1x128 scales [M][Nout/128];
    W_q stored [Nout][Nin] (contracted over its rows) with block scales
    sW [Nout/128][Nin/128] - the same table the forward pass uses."""
    Wt = np.ascontiguousarray(np.asarray(Wq, np.uint8).T)           # [Nin][Nout]
    sWt = np.ascontiguousarray(np.asarray(sW, np.float32).T)        # [Nin/128][Nout/128]
    return block_gemm(dYq, s_dY, Wt, expand_block_scales(sWt, Wt.shape[0]), with_magnitude)


def wgrad(dYq_t, s_dY_col, Xq_t, s_X_col, with_magnitude=False):
    """dW = dY^T X over tokens: dY_q^T [Nout][T] with 128x1 scales
    [Nout][T/128]; X_q^T [Nin][T] with 128x1 scales [Nin][T/128]."""
    return block_gemm(dYq_t, s_dY_col, Xq_t, s_X_col, with_magnitude)


def grouped_fprop(Xq, sX, offsets, Wq_e, sW_e, with_magnitude=False):
    """Per-expert Y_e = X_e W_e^T on row slices offsets[e]:offsets[e+1]."""
    offsets = np.asarray(offsets)
    outs, mags = [], []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        r = fprop(Xq[lo:hi], sX[lo:hi], Wq_e[e], sW_e[e], with_magnitude)
        if with_magnitude:
            outs.append(r[0]); mags.append(r[1])
        else:
            outs.append(r)
    R = np.concatenate(outs, axis=0)
    return (R, np.concatenate(mags, axis=0)) if with_magnitude else R


def round_to_bf16_bits(r) -> np.ndarray:
    """Round float64 values to BF16, nearest with ties to even; uint16 bits.

    BF16 keeps 8 significant bits: the spacing at magnitude 2**e (e >= -126)
    is 2**(e - 7), and 2**-133 below 2**-126.  Values at or beyond the
    midpoint above the largest finite BF16 round to infinity.  NaN -> 0x7FC0.
    """
    r = np.asarray(r, dtype=np.float64)
    nan = np.isnan(r)
    inf = np.isinf(r)
    rr = np.where(nan | inf, 0.0, r)
    _, ex = np.frexp(rr)                  # rr = m * 2**ex, 0.5 <= |m| < 1
    lead = ex - 1                         # exponent of the leading bit
    spacing_exp = np.maximum(lead - 7, -133)
    q = np.rint(np.ldexp(rr, -spacing_exp))             # exact scaling, then RNE
    v = np.ldexp(q, spacing_exp)
    v = np.where(np.abs(v) >= 2.0 ** 128, np.copysign(np.inf, rr), v)
    v = np.where(r == 0.0, np.copysign(0.0, r), v)
    v = np.where(inf, r, v)
    bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), bits).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(r) -> np.ndarray:
    """BF16 spacing at |r|: 2**(floor(log2|r|) - 7), floored at 2**-133."""
    r = np.abs(np.asarray(r, dtype=np.float64))
    _, ex = np.frexp(np.where(r == 0, 1.0, r))
    e = np.where(r == 0, -126, ex - 1)
    return np.ldexp(1.0, np.maximum(e - 7, -133))
