"""Fine-grained FP8 block-scaled quantization and GEMM for AMD MI355X (gfx950).

The compute lives in libfp8bs.so (HIP kernels behind a C ABI, declared in
include/fp8bs.h); this package loads it with ctypes and marshals PyTorch
tensors (device memory and the current stream).  Build the library with
``python -m fine_grained_fp8_amd.build``.  There is no CPU fallback: calls
fail loudly when the library is missing.
"""
from ._lib import FP8Error, load_library, LIB_PATH, SIGNATURES  # noqa: F401
from .ops import (  # noqa: F401
    quant_act_1x128,
    quant_act_dual,
    quant_weight_128x128,
    block_gemm,
    block_gemm_noalloc,
    block_gemm_fused_quant,
    block_gemm_grouped,
    amax_history_update,
    cast_e4m3,
    message_bytes,
    pack_tokens,
    unpack_tokens,
    dequant_tokens,
    gemm_promotion,
    quant_act_tiles,
    probe_mfma,
    probe_recip_online,
    probe_gemm_split,
    round_up,
)

__all__ = [
    "FP8Error", "load_library", "quant_act_1x128", "quant_act_dual", "quant_weight_128x128", "block_gemm",
    "block_gemm_noalloc", "block_gemm_fused_quant", "block_gemm_grouped", "amax_history_update", "cast_e4m3", "message_bytes", "pack_tokens",
    "unpack_tokens", "dequant_tokens", "gemm_promotion", "quant_act_tiles", "probe_mfma", "probe_recip_online", "probe_gemm_split", "round_up",
]
