"""GPU parity of the persistent GEMM's split-K tail.

When the output tiles leave the last round of one tile per workgroup at most
half full, the kernel cuts each leftover tile along K into pieces of whole
4-block rounds, run by workgroups that would otherwise idle; the piece that
finishes last adds the partial tiles in piece order and stores the tile.
These tests pick shapes where that happens at a size the oracle checks on
every row of the split tiles, confirm through the schedule query that the
launch did split, and check that the result does not depend on which piece
finishes last (two launches byte-identical).  The full-size Dgrad_T and
grouped tests in test_gpu_gemm.py run the same tail at the bench's shapes.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import gemm as og
from oracle import quant
from split_rule import persistent_grid, split_rule
from test_gpu_gemm import act_scales_dev, bf16_bits, dev, rows_one_per_tile, tiled_bytes
from tolerance import check_gemm, truncation_bound

pytestmark = pytest.mark.gpu


def expected_split(tiles, k_blocks, cus, slots=None):
    """The schedule rule of tests/split_rule.py on this device: the
    persistent grid from the CU count, the per-stream workspace of one
    partial tile per CU."""
    return split_rule(tiles, persistent_grid(tiles, cus), k_blocks, cus if slots is None else slots)


def device_cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_fprop_split_tail_ragged(gpu_lib, out_dtype):
    """Fprop 2100 x 3968 x 4096: 17 x 16 = 272 output tiles, the last row of
    tiles 52 rows high and the last column of tiles 128 wide.  On 256
    workgroups the 16 leftover tiles (that ragged last row of tiles, in the
    GroupM order) are cut into 8 pieces of 4 K blocks.  Every row of the split
    tiles and one row of every other M tile against the oracle; row-major and
    operand-tiled weights bit-identical; two launches byte-identical."""
    M, N, K = 2100, 3968, 4096
    tiles = ((M + 127) // 128) * ((N + 255) // 256)
    xb = syn.activation_with_outliers(M, K, seed=141)
    wb = syn.gaussian((N, K), seed=142, std=0.02)
    Xq, sX = quant.quant_rows(xb)
    Wq, sW = quant.quant_weight(wb)
    A, sA = dev(Xq), act_scales_dev(sX)
    C = gpu_lib.block_gemm("fprop", A, sA, dev(Wq), dev(sW), out_dtype=out_dtype)
    Ct = gpu_lib.block_gemm("fprop_tiled", A, sA, dev(tiled_bytes(Wq)), dev(sW), out_dtype=out_dtype)
    Ct2 = gpu_lib.block_gemm("fprop_tiled", A, sA, dev(tiled_bytes(Wq)), dev(sW), out_dtype=out_dtype)
    torch.cuda.synchronize()
    n_split, pieces = gpu_lib.probe_gemm_split(tiles, K)
    assert (n_split, pieces) == expected_split(tiles, K // 128, device_cus())
    if device_cus() == 256:
        assert (n_split, pieces) == (16, 8)
    assert n_split > 0, "the launch must exercise the split tail"
    view = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    assert torch.equal(C.view(view), Ct.view(view)), "tiled and row-major differ"
    assert torch.equal(Ct.view(view), Ct2.view(view)), "two launches differ"
    rows = np.unique(np.concatenate([rows_one_per_tile(M, seed=143), np.arange(2048, M)]))
    R, T = og.fprop(Xq[rows], sX[rows], Wq, sW, with_magnitude=True)
    E = truncation_bound(Xq[rows], sX[rows], Wq, og.expand_block_scales(sW, N))
    y = C.cpu().numpy()[rows] if out_dtype == torch.float32 else bf16_bits(C)[rows]
    check_gemm(y, R, T, K, out="fp32" if out_dtype == torch.float32 else "bf16", E=E,
               label=f"fprop split tail 2100x3968x4096 {'fp32' if out_dtype == torch.float32 else 'bf16'}")


def test_wgrad_split_tail(gpu_lib):
    """Wgrad (FP32 out, rank-1 scale fold) 2304 x 3840 x 1280: 18 x 15 = 270
    tiles, 14 left over on 256 workgroups, cut into pieces of one 4-block
    round (K = 1280 tokens: 10 blocks, 3 rounds, the last one padded).  Every
    row of the split tiles and one row of every M tile against the oracle;
    two launches byte-identical."""
    D_out, D_in, Tk = 2304, 3840, 1280
    tiles = (D_out // 128) * (D_in // 256)
    dyb = syn.gaussian((Tk, D_out), seed=151, std=1e-3)
    xb = syn.activation_with_outliers(Tk, D_in, seed=152)
    dYt, s_dy = quant.quant_cols(dyb)
    Xt, s_x = quant.quant_cols(xb)
    A, sA, B, sB = dev(dYt), act_scales_dev(s_dy), dev(Xt), act_scales_dev(s_x)
    C = gpu_lib.block_gemm("wgrad", A, sA, B, sB, out_dtype=torch.float32)
    C2 = gpu_lib.block_gemm("wgrad", A, sA, B, sB, out_dtype=torch.float32)
    torch.cuda.synchronize()
    n_split, pieces = gpu_lib.probe_gemm_split(tiles, Tk)
    assert (n_split, pieces) == expected_split(tiles, Tk // 128, device_cus())
    assert n_split > 0, "the launch must exercise the split tail"
    assert torch.equal(C.view(torch.int32), C2.view(torch.int32)), "two launches differ"
    # the leftover tiles are the last `n_split` in the GroupM order; take
    # every row of the M tiles they lie in
    tiles_m, tiles_n = D_out // 128, D_in // 256
    split_m = set()
    for b in range(tiles - n_split, tiles):
        grp = b // (8 * tiles_n)
        gsz = min(8, tiles_m - grp * 8)
        split_m.add(grp * 8 + (b - grp * 8 * tiles_n) % gsz)
    rows = np.unique(np.concatenate([rows_one_per_tile(D_out, seed=153)] +
                                    [np.arange(128 * m, 128 * m + 128) for m in sorted(split_m)]))
    R, T = og.wgrad(dYt[rows], s_dy[rows], Xt, s_x, with_magnitude=True)
    E = truncation_bound(dYt[rows], s_dy[rows], Xt, s_x)
    check_gemm(C.cpu().numpy()[rows], R, T, Tk, out="fp32", E=E, label="wgrad split tail 2304x3840x1280")


def test_full_size_schedules_split_where_the_bench_runs(gpu_lib):
    """The bench's shapes on this device: Fprop (2304 tiles) and Wgrad (4032)
    run whole tiles only; Dgrad_T (896 tiles, K 18432) and the config-5
    grouped launch (1048 tiles, K 7168) split their leftover tiles - the
    full-size parity tests of those two run through the split tail."""
    cus = device_cus()
    counts = syn.expert_counts(16384, 8, seed=0)
    grouped_tiles = int(sum((int(c) + 127) // 128 for c in counts)) * 8
    cases = {"fprop": (2304, 7168), "wgrad": (4032, 4096), "dgrad_t": (896, 18432), "grouped": (grouped_tiles, 7168)}
    # the current stream's split workspace exists once any GEMM ran on it
    Xq, sX = quant.quant_rows(syn.gaussian((128, 128), seed=161))
    Wq, sW = quant.quant_weight(syn.gaussian((256, 128), seed=162, std=0.02))
    gpu_lib.block_gemm("fprop", dev(Xq), act_scales_dev(sX), dev(Wq), dev(sW))
    torch.cuda.synchronize()
    for name, (tiles, K) in cases.items():
        got = gpu_lib.probe_gemm_split(tiles, K)
        assert got == expected_split(tiles, K // 128, cus), name
    if cus == 256:
        assert gpu_lib.probe_gemm_split(2304, 7168) == (0, 1)
        assert gpu_lib.probe_gemm_split(4032, 4096) == (0, 1)
        assert gpu_lib.probe_gemm_split(896, 18432) == (128, 2)
        assert gpu_lib.probe_gemm_split(grouped_tiles, 7168) == (grouped_tiles % 256, 7)
