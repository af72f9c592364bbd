"""The pages' worked examples, computed with the oracle (test infrastructure only).

* ``two_tiles`` - "Fine-Grained FP8 Quantization in DeepSeek", worked example:
  one 128-value tile centred near 0.1 and one containing a 20.0 outlier;
  reconstruction error under one global scale versus one scale per tile, and
  scale bytes per activation value.
* ``per_tensor_vs_fine`` - "FP8 Mixed Precision: DeepSeek-V3 Training
  Architecture", Step 2: 64 tokens x 512 channels of 0.4 * N(0, 1) with +35
  added to channel 88, weights 1024 x 512 of 0.08 * N(0, 1) (legacy numpy
  seed 42, kept as cited data); relative Frobenius error of the GEMM with one
  scale per tensor versus 1x128 / 128x128 scales, computed with the oracle's
  quantizers and block GEMM.  Codes are on the E4M3 grid here (the page's
  simulation rounds to integers instead).
"""
from __future__ import annotations

import numpy as np

from . import e4m3, quant


def _groups_quant(x32: np.ndarray):
    """Quantize float32 groups x32[..., n]; return float64 reconstruction and scales."""
    q, s, _, _ = quant._quantize_groups(x32)
    return e4m3.decode(q) * s.astype(np.float64)[..., None], s


def two_tiles(seed: int = 0):
    """Tile A ~ 0.1 + 0.01 N(0,1); tile B the same with element 0 = 20.0 (BF16)."""
    rng = np.random.default_rng(seed)
    a = (0.1 + 0.01 * rng.standard_normal(128)).astype(np.float32)
    b = (0.1 + 0.01 * rng.standard_normal(128)).astype(np.float32)
    b[0] = 20.0
    tiles = quant.bf16_to_f32(_f32_to_bf16(np.stack([a, b])))       # [2][128]
    glob, s_glob = _groups_quant(tiles.reshape(1, 256))
    loc, s_loc = _groups_quant(tiles)
    x = tiles.astype(np.float64)
    glob = glob.reshape(2, 128)

    def rms_rel(rec, ref):
        return float(np.sqrt(np.mean(((rec - ref) / ref) ** 2)))

    return dict(
        tiles=tiles, s_global=s_glob[0], s_local=s_loc,
        q_global=e4m3.encode((tiles / s_glob[0]).astype(np.float32)),
        q_local=e4m3.encode((tiles / s_loc[:, None]).astype(np.float32)),
        err_global=[rms_rel(glob[i], x[i]) for i in range(2)],
        err_local=[rms_rel(loc[i], x[i]) for i in range(2)],
        abs_err_global=np.abs(glob - x), abs_err_local=np.abs(loc - x),
        scale_bytes_per_value_global=4 / 256,
        scale_bytes_per_value_local=4 / 128,
    )


def per_tensor_vs_fine():
    """Relative GEMM error, per-tensor vs fine-grained scales, on the E4M3 grid.

    The data are the page's fixture (its Step 2 values, kept as data): legacy
    numpy seed 42, X = 0.4 N(0, 1) of 64 tokens x 512 channels with +35 on
    channel 88, W = 0.08 N(0, 1) of 1024 x 512, both rounded to BF16 (the
    method quantizes BF16 tensors).  Both quantizations and both GEMMs come
    from the oracle's own functions: fine-grained = quant_rows (1x128) and
    quant_weight (128x128) into gemm.fprop; per-tensor = the same codec with
    one scale for the whole tensor (quant_rows_external with every tile's
    scale equal), which the block GEMM applies exactly like a per-tensor
    scale.  The reference is the float64 product of the BF16 inputs.
    """
    from . import gemm as og
    rs = np.random.RandomState(42)
    X = rs.randn(64, 512) * 0.4
    X[:, 88] += 35.0
    W = rs.randn(1024, 512) * 0.08
    Xb, Wb = _f32_to_bf16(X.astype(np.float32)), _f32_to_bf16(W.astype(np.float32))
    Y_ref = quant.bf16_to_f32(Xb).astype(np.float64) @ quant.bf16_to_f32(Wb).astype(np.float64).T
    # fine-grained: 1x128 activation tiles, 128x128 weight blocks
    Xq, sX = quant.quant_rows(Xb)
    Wq, sW = quant.quant_weight(Wb)
    Y_f = og.fprop(Xq, sX, Wq, sW)
    # per-tensor: one scale from each tensor's max
    sx = quant.scale_from_amax(np.max(np.abs(quant.bf16_to_f32(Xb))))
    sw = quant.scale_from_amax(np.max(np.abs(quant.bf16_to_f32(Wb))))
    Xq_t, _, _ = quant.quant_rows_external(Xb, np.full((64, 4), sx, np.float32))
    Wq_t, _, _ = quant.quant_rows_external(Wb, np.full((1024, 4), sw, np.float32))
    Y_t = og.fprop(Xq_t, np.full((64, 4), sx, np.float32), Wq_t, np.full((8, 4), sw, np.float32))
    err_t = np.linalg.norm(Y_t - Y_ref) / np.linalg.norm(Y_ref)
    err_f = np.linalg.norm(Y_f - Y_ref) / np.linalg.norm(Y_ref)
    return dict(err_per_tensor=float(err_t), err_fine=float(err_f))


def _f32_to_bf16(x):
    b = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
