"""fp8_block_gemm_noalloc (the GEMM entry point that allocates nothing, its
split workspace a static device array) against fp8_block_gemm on the same
inputs: bit-identical outputs on two calls in a row, the second smaller,
both at shapes whose leftover tiles are split along K (so the static
workspace and its counters are exercised, and the second call runs on the
array the first one left behind)."""
import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import quant

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def act_scales_dev(s_rows):
    M, KB = s_rows.shape
    buf = np.zeros((KB, (M + 3) // 4 * 4), np.float32)
    buf[:, :M] = s_rows.T
    return dev(buf)


def test_noalloc_matches_block_gemm_on_two_calls(gpu_lib):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus > 256:
        pytest.skip("the static split workspace holds 256 pieces")
    cases = [("fprop", 2100, 3968, 4096, torch.bfloat16, 201),    # 272 tiles: 16 split into 8
             ("fprop", 1100, 7680, 2048, torch.float32, 202)]     # 270 tiles: 14 split into 4, smaller input
    for layout, M, N, K, out_dtype, seed in cases:
        Xq, sX = quant.quant_rows(syn.activation_with_outliers(M, K, seed=seed))
        Wq, sW = quant.quant_weight(syn.gaussian((N, K), seed=seed + 1, std=0.02))
        A, sA, B, sB = dev(Xq), act_scales_dev(sX), dev(Wq), dev(sW)
        ref = gpu_lib.block_gemm(layout, A, sA, B, sB, out_dtype=out_dtype)
        out = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
        gpu_lib.block_gemm_noalloc(layout, A, sA, B, sB, out=out)
        torch.cuda.synchronize()
        tiles = ((M + 127) // 128) * ((N + 255) // 256)
        n_split, pieces = gpu_lib.probe_gemm_split(tiles, K)
        if cus == 256:
            assert n_split > 0 and pieces >= 2, (layout, M, N, K)
        view = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
        assert torch.equal(out.view(view), ref.view(view)), (layout, M, N, K)
