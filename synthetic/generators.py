"""Seeded input generators (no quantization or GEMM arithmetic lives here).

Distributions follow the workloads the pages describe for fine-grained FP8:
Gaussian activations whose outliers concentrate in a few fixed channels
("Fine-Grained FP8 Quantization in DeepSeek", failure-modes list: Gaussian-only
tests under-represent outliers), Gaussian weights, small Gaussian gradients,
a tile whose spread doubles over 100 steps with one rare 20-sigma spike
("Online Quantization During Training", worked example), and per-expert
token counts for the grouped expert GEMM.
"""
from __future__ import annotations

import numpy as np

# Shapes of the five workloads (rows x cols, row-major).  Hidden size 7168,
# dense FFN width 18432 and expert FFN width 2048 are DeepSeek-V3-like.
CONFIGS = {
    "toy": dict(M=128, K=128, N=256),
    "quantizer": dict(M=8192, K=7168),
    "drift": dict(steps=100, M=128, K=7168, spike_step=50),
    "fprop": dict(M=4096, K=7168, N=18432),
    "backward": dict(M=4096, d_in=7168, d_out=18432),
    "grouped": dict(tokens=16384, experts=8, K=7168, N=2048),
}


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to BF16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(u16) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (exact)."""
    u = np.ascontiguousarray(u16, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def gaussian(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """BF16 bits of std * N(0, 1) with a seeded generator."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def activation_with_outliers(M: int, K: int, seed: int, n_channels: int = 16,
                             frac: float = 1e-3, magnitude: float = 20.0) -> np.ndarray:
    """BF16 bits of N(0, 1) activations with channel-concentrated outliers.

    ``round(frac * M * K)`` cells, drawn without replacement from the
    ``M x n_channels`` grid of (row, outlier-channel) pairs, are set to
    ``+-magnitude`` with a seeded random sign.  The outlier channels are drawn
    once, without replacement, from the K channels.
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    n_channels = min(n_channels, K)
    channels = rng.choice(K, size=n_channels, replace=False)
    cap = M * n_channels
    n_out = min(int(round(frac * M * K)), cap)
    if n_out > 0:
        cells = rng.choice(cap, size=n_out, replace=False)
        rows = cells // n_channels
        cols = channels[cells % n_channels]
        signs = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=n_out)
        x[rows, cols] = signs * np.float32(magnitude)
    return f32_to_bf16_bits(x)


def toy_layer(seed: int = 0):
    """The toy linear layer y = W x widened to 128 tokens.

    X: 128 x 128 ~ N(0, 1) with element (0, 42) set to 20.0; W: 256 x 128 ~
    N(0, 0.02).  Returns (X_bits, W_bits).
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((128, 128), dtype=np.float32)
    x[0, 42] = 20.0
    w = rng.standard_normal((256, 128), dtype=np.float32) * np.float32(0.02)
    return f32_to_bf16_bits(x), f32_to_bf16_bits(w)


def drift_sequence(steps: int = 100, M: int = 128, K: int = 7168, seed: int = 0,
                   spike_step: int = 50, spike_sigma: float = 20.0):
    """Yield (t, sigma_t, X_t bits) for a tile whose std doubles linearly.

    sigma_t = 1 + t / (steps - 1); at ``spike_step`` one seeded element is set
    to +-spike_sigma * sigma_t.
    """
    pos_rng = np.random.default_rng([seed, 1_000_003])
    spike_row = int(pos_rng.integers(M))
    spike_col = int(pos_rng.integers(K))
    spike_sign = float(pos_rng.choice([-1.0, 1.0]))
    for t in range(steps):
        sigma = 1.0 + t / (steps - 1)
        rng = np.random.default_rng([seed, t])
        x = rng.standard_normal((M, K), dtype=np.float32) * np.float32(sigma)
        if t == spike_step:
            x[spike_row, spike_col] = np.float32(spike_sign * spike_sigma * sigma)
        yield t, sigma, f32_to_bf16_bits(x)


def curriculum_sequence(steps: int = 100, M: int = 128, K: int = 7168, seed: int = 0,
                        shifts=((40, 4.0), (70, 1.0))):
    """Yield (t, sigma_t, X_t bits) for a data mix that changes abruptly.

    sigma_t = 1 until the first shift step, then the factor of the latest
    shift reached (default: 4x from step 40, back to 1x from step 70);
    X_t = sigma_t N(0, 1), a fresh seeded draw per step.
    """
    for t in range(steps):
        sigma = 1.0
        for step, factor in shifts:
            if t >= step:
                sigma = float(factor)
        rng = np.random.default_rng([seed, 7, t])
        x = rng.standard_normal((M, K), dtype=np.float32) * np.float32(sigma)
        yield t, sigma, f32_to_bf16_bits(x)


def expert_counts(tokens: int = 16384, experts: int = 8, seed: int = 0) -> np.ndarray:
    """Per-expert token counts from a seeded uniform multinomial."""
    rng = np.random.default_rng(seed)
    return rng.multinomial(tokens, [1.0 / experts] * experts).astype(np.int64)


def expert_offsets(counts) -> np.ndarray:
    """int32 prefix sums [0, n_0, n_0 + n_1, ...] (len = experts + 1)."""
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def dispatch_rows(tokens: int, experts: int, topk: int, seed: int = 0) -> np.ndarray:
    """Source token of every dispatched copy, grouped by expert.

    Each token picks ``topk`` distinct experts uniformly at random (seeded);
    the copies are listed expert by expert, tokens ascending within an expert.
    Returns int32 [tokens * topk].
    """
    rng = np.random.default_rng(seed)
    choice = np.argsort(rng.random((tokens, experts)), axis=1)[:, :topk]   # distinct experts
    tok = np.repeat(np.arange(tokens), topk)
    exp = choice.reshape(-1)
    order = np.lexsort((tok, exp))
    return tok[order].astype(np.int32)


def lossless_tiles(rows: int, cols: int, seed: int, tile=(1, 128), k_range=(-30, 20)):
    """BF16 bits whose every scaling tile is exactly representable.

    Each tile (``tile`` = (tile_rows, tile_cols), anchored at (0, 0)) gets a
    power of two 2**k (k drawn per tile from ``k_range``); its elements are
    ``n * 2**j * 2**k`` with n in 0..15 and j in -9..4 (at most four
    significant bits, magnitude at most 448), and one element per tile is
    +-448 * 2**k.  Returns (bits, k) with k shaped (rows / tr, cols / tc).
    """
    tr, tc = tile
    assert rows % tr == 0 and cols % tc == 0
    rng = np.random.default_rng(seed)
    n = rng.integers(0, 16, size=(rows, cols))
    j = rng.integers(-9, 5, size=(rows, cols))
    v = n.astype(np.float64) * np.exp2(j)
    v = np.where(v > 448.0, v / 2.0, v)
    v *= rng.choice([-1.0, 1.0], size=(rows, cols))
    kt = rng.integers(k_range[0], k_range[1] + 1, size=(rows // tr, cols // tc))
    # one +-448 per tile at a seeded position
    pr = rng.integers(0, tr, size=kt.shape)
    pc = rng.integers(0, tc, size=kt.shape)
    ps = rng.choice([-1.0, 1.0], size=kt.shape)
    ti, tj = np.meshgrid(np.arange(kt.shape[0]), np.arange(kt.shape[1]), indexing="ij")
    v[ti * tr + pr, tj * tc + pc] = 448.0 * ps
    k_full = np.repeat(np.repeat(kt, tr, axis=0), tc, axis=1)
    x = (v * np.exp2(k_full)).astype(np.float32)
    return f32_to_bf16_bits(x), kt
