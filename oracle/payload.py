"""FP8 token payloads for activation caching and MoE dispatch (oracle; test
infrastructure only).

Sources:

* "FP8 Mixed Precision: DeepSeek-V3 Training Architecture", section 4
  (low-precision systems co-design): activations kept for the backward pass
  are stored in FP8, and the token representations sent to remote experts in
  the MoE all-to-all are quantized to FP8 on the fly; its section on the MoE
  all-to-all communication wall: each dispatched token is one hidden vector,
  sent to the expert's GPU and combined back.
* "Fine-Grained FP8 Quantization in DeepSeek", section 2: the 1x128 tile scale
  travels with the tile's codes.

Readings taken where the pages leave a step open:

* A token's message is its 1x128-quantized hidden vector (``quant.quant_rows``
  of that one row) in a self-contained byte layout: the H E4M3 codes, then
  the H/128 FP32 scales, little-endian, in tile order.  H + 4 H / 128 bytes.
  Messages sit at a caller-chosen byte stride.
* Packing may gather: message t carries source row src_rows[t] (the dispatch
  order).  A source row outside the input gives a message of NaN codes (0x7F)
  and NaN scales (0x7FC00000), which any consumer sees.
* Restoring BF16 from a message is x = q * s rounded once to BF16 (nearest,
  ties to even): the product of an E4M3 value (4 significant bits) and an
  FP32 scale (24) is exact in float64, so only the final rounding remains.
"""
from __future__ import annotations

import numpy as np

from . import e4m3, quant
from .gemm import round_to_bf16_bits

TILE = 128


def message_bytes(H: int) -> int:
    """Bytes of one token message: H codes + H/128 FP32 scales."""
    assert H % TILE == 0
    return H + 4 * (H // TILE)


def pack_tokens(x_bits, src_rows=None, stride: int | None = None) -> np.ndarray:
    """BF16 tokens [rows][H] -> messages uint8 [T][stride]; bytes past the
    message are zero.  T = len(src_rows) (default: every row in order)."""
    x_bits = np.asarray(x_bits, np.uint16)
    rows, H = x_bits.shape
    mb = message_bytes(H)
    stride = mb if stride is None else stride
    assert stride >= mb
    src = np.arange(rows) if src_rows is None else np.asarray(src_rows, np.int64)
    T = len(src)
    out = np.zeros((T, stride), np.uint8)
    ok = (src >= 0) & (src < rows)
    if ok.any():
        q, s = quant.quant_rows(x_bits[src[ok]])            # q [n][H], s [n][H/128]
        out[ok, :H] = q
        out[ok, H:mb] = np.ascontiguousarray(s.astype("<f4")).view(np.uint8).reshape(-1, mb - H)
    bad = ~ok
    if bad.any():
        out[bad, :H] = 0x7F
        nan = np.full((H // TILE,), np.uint32(0x7FC00000), "<u4").view(np.uint8)
        out[bad, H:mb] = nan
    return out


def unpack_tokens(msgs, H: int):
    """Messages -> (codes uint8 [T][H], scales float32 [T][H/128])."""
    m = np.asarray(msgs, np.uint8)
    mb = message_bytes(H)
    q = np.ascontiguousarray(m[:, :H])
    s = np.ascontiguousarray(m[:, H:mb]).view("<f4").astype(np.float32).reshape(m.shape[0], H // TILE)
    return q, s


def dequant_tokens(msgs, H: int) -> np.ndarray:
    """Messages -> BF16 bits [T][H]: RNE_bf16(q * s), the product exact in float64."""
    q, s = unpack_tokens(msgs, H)
    v = e4m3.decode(q) * np.repeat(s.astype(np.float64), TILE, axis=1)
    return round_to_bf16_bits(v)
