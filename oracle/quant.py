"""Fine-grained FP8 quantization (oracle; test infrastructure only).

Sources:

* "Fine-Grained FP8 Quantization in DeepSeek", sections 2 (activations: one scale
  per tile of 128 contiguous values) and 3 (weights: one scale per 128x128
  block).
* "FP8 Mixed Precision: DeepSeek-V3 Training Architecture", section 1: the
  1x128 tiles run along the channel dimension of each token; the block scale
  is the block's max |value| divided by 448 and the quantized value is the
  scaled value clipped to [-448, 448]; its Step 1 code floors the scale at
  1e-12 and anchors tiles/blocks at index 0 with divisibility asserts.
* "Introduction to LLM Quantization", section 5 (online quantization): the
  max |value| of each 1x128 tile or 128x128 block is computed on the fly,
  turned into a scale at once, and the tensor is quantized with it.

Readings taken where the pages leave a step open:

* Codes are on the E4M3 grid (``oracle.e4m3``), not the integer grid the
  page's simulation rounds to: the format is E4M3 throughout.
* Arithmetic is FP32 with IEEE round-to-nearest: s = fl32(amax / 448),
  s = max(s, fl32(1e-12)); q = E4M3(fl32(x / s)).  The quotient is a true
  division by s (not a multiplication by 1/s); the stored scale is s, the
  dequantization multiplier (x ~ q * s).
* A tile containing NaN has amax NaN and scale NaN (stored as the canonical
  quiet NaN 0x7FC00000); every code of the tile is then NaN (0x7F).  A tile
  containing +-Inf (no NaN) has scale Inf: finite elements give +-0 codes and
  infinite ones give NaN (Inf / Inf).
* 128x1 column tiles (weight-gradient operands) are the 1x128 rule applied
  to the transpose, with the transposed codes as output.

Input convention: activations and weights arrive as BF16 bit patterns
(uint16 arrays); BF16 -> FP32 widening is exact.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

TILE = 128
E4M3_MAX = np.float32(448.0)
SCALE_FLOOR = np.float32(1e-12)                  # bits 0x2B8CBCCC
CANONICAL_NAN = np.uint32(0x7FC00000).view(np.float32)
# The page's weight equation rounds first and clips the rounded value to
# [-448, 448].  On the E4M3 grid extended past 448 the next value is 480, so a
# scaled value is changed by the clip (saturated) exactly when its magnitude
# exceeds the midpoint 464 (464 itself ties to 448, the even code).
CLIP_THRESHOLD = np.float32(464.0)


def bf16_to_f32(bits) -> np.ndarray:
    """BF16 bit patterns -> float32 (exact: BF16 is the top half of FP32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def scale_from_amax(amax) -> np.ndarray:
    """s = max(fl32(amax / 448), fl32(1e-12)); NaN amax -> canonical NaN."""
    amax = np.asarray(amax, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        s = (amax / E4M3_MAX).astype(np.float32)
        s = np.maximum(s, SCALE_FLOOR).astype(np.float32)
    return np.where(np.isnan(s), CANONICAL_NAN, s).astype(np.float32)


def _quantize_groups(xg: np.ndarray, scales=None):
    """Quantize float32 groups xg[..., n] with one scale per group.

    Returns (codes uint8 like xg, scale float32 xg.shape[:-1],
    amax float32, saturated-count int).
    """
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        amax = np.max(np.abs(xg), axis=-1).astype(np.float32)   # NaN propagates
        s = scale_from_amax(amax) if scales is None else np.asarray(scales, np.float32)
        y = (xg / s[..., None]).astype(np.float32)               # IEEE fl32 division
    codes = e4m3.encode(y)
    saturated = int(np.count_nonzero(np.abs(y) > CLIP_THRESHOLD))  # NaN compares false
    return codes, s.astype(np.float32), amax, saturated


def quant_rows(x_bits):
    """1x128 activation tiles along the columns of each row.

    x_bits: uint16 [M][K], K % 128 == 0.
    Returns (q uint8 [M][K], s float32 [M][K/128]).
    """
    x = bf16_to_f32(x_bits)
    M, K = x.shape
    assert K % TILE == 0, "K must be a multiple of 128"
    q, s, _, _ = _quantize_groups(x.reshape(M, K // TILE, TILE))
    return q.reshape(M, K), s


def quant_cols(x_bits):
    """128x1 tiles along the rows (tokens), output transposed.

    x_bits: uint16 [M][C], M % 128 == 0.
    Returns (q_t uint8 [C][M], s float32 [C][M/128]) - the row rule on x^T.
    """
    xt = np.ascontiguousarray(np.asarray(x_bits, dtype=np.uint16).T)
    assert xt.shape[1] % TILE == 0, "M must be a multiple of 128"
    return quant_rows(xt)


def quant_weight(w_bits):
    """128x128 weight blocks anchored at (0, 0).

    w_bits: uint16 [N][K], N % 128 == K % 128 == 0.
    Returns (q uint8 [N][K], s float32 [N/128][K/128]).
    """
    w = bf16_to_f32(w_bits)
    N, K = w.shape
    assert N % TILE == 0 and K % TILE == 0, "both weight dims must be multiples of 128"
    nb, kb = N // TILE, K // TILE
    blocks = w.reshape(nb, TILE, kb, TILE).transpose(0, 2, 1, 3).reshape(nb, kb, TILE * TILE)
    q, s, _, _ = _quantize_groups(blocks)
    q = q.reshape(nb, kb, TILE, TILE).transpose(0, 2, 1, 3).reshape(N, K)
    return q, s


def quant_rows_external(x_bits, scales):
    """1x128 row tiles with caller-supplied scales (delayed/static policies).

    scales: float32 [M][K/128].  Returns (q uint8 [M][K], amax float32
    [M][K/128], saturated) where ``saturated`` counts elements the clip
    changes: scaled value fl32(x / s) with magnitude above 464 (Inf included,
    NaN not).
    """
    x = bf16_to_f32(x_bits)
    M, K = x.shape
    assert K % TILE == 0
    q, _, amax, sat = _quantize_groups(x.reshape(M, K // TILE, TILE), scales)
    return q.reshape(M, K), amax, sat


def dequant_rows(q, s) -> np.ndarray:
    """float64 reconstruction q * s for 1x128 row tiles (exact in float64)."""
    q = np.asarray(q, dtype=np.uint8)
    M, K = q.shape
    v = e4m3.decode(q).reshape(M, K // TILE, TILE)
    return (v * np.asarray(s, np.float64)[..., None]).reshape(M, K)


def dequant_weight(q, s) -> np.ndarray:
    """float64 reconstruction of 128x128-block-quantized weights."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    full = np.repeat(np.repeat(np.asarray(s, np.float64), TILE, axis=0), TILE, axis=1)
    return e4m3.decode(q) * full
