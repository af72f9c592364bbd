"""GPU parity of the Fprop GEMM with the 1x128 quantization of X fused in.

The fused kernel must form exactly the 1x128 quantizer's codes and scales
(so its output equals the unfused quantizer + GEMM bit for bit) and stay
within the GEMM tolerance of the float64 oracle.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import gemm as og
from oracle import quant
from tolerance import check_gemm, truncation_bound, truncation_bound_at

pytestmark = pytest.mark.gpu

BF16_INF, BF16_NAN = 0x7F80, 0x7FC0


def dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.cuda()


@pytest.mark.parametrize("case", ["ragged", "fp32_out", "many_tiles", "inf_nan"])
def test_fused_quant_fprop_equals_quant_then_gemm(gpu_lib, case):
    rows, depth, cols = {"ragged": (333, 640, 640), "fp32_out": (333, 640, 640),
                         "many_tiles": (1100, 1152, 768), "inf_nan": (200, 384, 256)}[case]
    out_dtype = torch.float32 if case == "fp32_out" else torch.bfloat16
    xb = syn.activation_with_outliers(rows, depth, seed=111)
    wb = syn.gaussian((cols, depth), seed=112, std=0.02)
    if case == "inf_nan":
        xb = xb.copy()
        xb[3, 5] = BF16_INF                 # an infinite tile (scale Inf)
        xb[17, 300] = BF16_NAN              # a NaN tile (scale NaN)
    Wq, sW = quant.quant_weight(wb)
    x = dev(xb)
    C, q, s = gpu_lib.block_gemm_fused_quant(x, dev(Wq), dev(sW), out_dtype=out_dtype, with_codes=True)
    qu, su, _ = gpu_lib.quant_act_1x128(x, "row")
    Cu = gpu_lib.block_gemm("fprop", qu, su, dev(Wq), dev(sW), out_dtype=out_dtype)
    torch.cuda.synchronize()
    # the codes and scales the kernel formed are the quantizer's
    assert torch.equal(q, qu)
    assert torch.equal(s[:, :rows].view(torch.int32), su[:, :rows].view(torch.int32))
    # and so is the product, bit for bit (NaN rows included)
    view = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    assert torch.equal(C.view(view), Cu.view(view))
    if case == "inf_nan":
        return
    # pinned to the oracle as well
    Xq, sX = quant.quant_rows(xb)
    assert np.array_equal(q.cpu().numpy(), Xq)
    R, T = og.fprop(Xq, sX, Wq, sW, with_magnitude=True)
    E = truncation_bound(Xq, sX, Wq, og.expand_block_scales(sW, cols))
    if out_dtype == torch.float32:
        check_gemm(C.cpu().numpy(), R, T, depth, out="fp32", E=E, label=f"fused {case}")
    else:
        check_gemm(C.view(torch.int16).cpu().numpy().view(np.uint16), R, T, depth, E=E, label=f"fused {case}")


def test_fused_quant_fprop_without_codes(gpu_lib):
    xb = syn.activation_with_outliers(256, 512, seed=113)
    wb = syn.gaussian((256, 512), seed=114, std=0.02)
    Wq, sW = quant.quant_weight(wb)
    x = dev(xb)
    C = gpu_lib.block_gemm_fused_quant(x, dev(Wq), dev(sW))
    qu, su, _ = gpu_lib.quant_act_1x128(x, "row")
    Cu = gpu_lib.block_gemm("fprop", qu, su, dev(Wq), dev(sW))
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), Cu.view(torch.int16))


def test_fused_quant_fprop_full_size(gpu_lib, big_layer):
    """The bench's layer at full size (X 4096x7168 with outliers, W_q
    18432x7168): the codes and scales the fused kernel forms equal the
    oracle's, its output equals quantize-then-GEMM bit for bit, and one row
    per M tile is checked against the oracle."""
    Xq, sX, Wq, sW = big_layer
    xb = syn.activation_with_outliers(4096, 7168, seed=0)
    x = dev(xb)
    del xb
    W, S = dev(Wq), dev(sW)
    C, q, s = gpu_lib.block_gemm_fused_quant(x, W, S, with_codes=True)
    qu, su, _ = gpu_lib.quant_act_1x128(x, "row")
    Cu = gpu_lib.block_gemm("fprop", qu, su, W, S)
    torch.cuda.synchronize()
    assert torch.equal(q, qu)
    assert torch.equal(s[:, :4096].view(torch.int32), su[:, :4096].view(torch.int32))
    assert torch.equal(C.view(torch.int16), Cu.view(torch.int16))
    assert np.array_equal(q.cpu().numpy(), Xq)
    assert np.array_equal(s[:, :4096].cpu().numpy().T.view(np.uint32), sX.view(np.uint32))
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, 4095], np.arange(0, 4096, 128) + rng.integers(0, 128, 32)]))
    R, T = og.fprop(Xq[rows], sX[rows], Wq, sW, with_magnitude=True)
    sWn = og.expand_block_scales(sW, 18432)
    check_gemm(C.view(torch.int16).cpu().numpy().view(np.uint16)[rows], R, T, 7168,
               label="fused quant+fprop 4096x18432x7168",
               E_at=lambda r, c: truncation_bound_at(Xq[rows], sX[rows], Wq, sWn, r, c))
