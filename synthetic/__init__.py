"""Seeded synthetic inputs shared by the tests, the bench and the smoke run.

This module produces the input tensors only: Gaussian activations with
channel-concentrated outliers, Gaussian weights and gradients, the drifting
tile sequence of the online-scaling worked example, expert token counts and
the dispatch order of routed token copies, and a tile sequence whose
distribution jumps (a curriculum change).
It holds none of the quantization or GEMM arithmetic; the oracle and the HIP
path both consume what it returns.

Every tensor comes back as BF16 bit patterns (``numpy.uint16``), rounded to
nearest-even from the FP32 draw, so the oracle and the GPU see the same bytes.
"""
from .generators import (  # noqa: F401
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    activation_with_outliers,
    gaussian,
    toy_layer,
    drift_sequence,
    curriculum_sequence,
    expert_counts,
    expert_offsets,
    dispatch_rows,
    lossless_tiles,
    CONFIGS,
)
