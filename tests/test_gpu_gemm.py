"""GPU parity of the block-scaled FP8 GEMMs against the float64 oracle.

Operands are quantized by the ORACLE (so the GEMM check does not depend on
the GPU quantizers) and uploaded; the GPU result is compared elementwise with
``tests/tolerance.py``'s bar.  Full-size cases run the whole GEMM in the
configuration the bench times and compare a seeded sample of output rows.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import gemm as og
from oracle import quant
from tolerance import check_gemm, truncation_bound, truncation_bound_at

pytestmark = pytest.mark.gpu


def dev(a):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a)
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.cuda()


def act_scales_dev(s_rows):
    """oracle [M][K/128] -> device MN-major [K/128][round_up(M, 4)]."""
    M, KB = s_rows.shape
    buf = np.zeros((KB, (M + 3) // 4 * 4), np.float32)
    buf[:, :M] = s_rows.T
    return dev(buf)


def bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def rows_one_per_tile(M, seed, tile=128):
    """One seeded row in every 128-row tile of an M-row output, plus the first
    and the last row: every M tile of the launch is sampled."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, M, tile)
    picks = starts + rng.integers(0, np.minimum(tile, M - starts))
    return np.unique(np.concatenate([[0, M - 1], picks]))


def tiled_bytes(q):
    """Operand-tiled bytes of row-major codes q [R][C] (R % 16 == 0,
    C % 128 == 0), returned in a [R][C] array: oracle.tiling's layout written
    as one reshape (pinned to tiling.tile_codes in
    test_tiled_bytes_reshape_matches_the_oracle_layout)."""
    R, C = q.shape
    t = np.asarray(q, np.uint8).reshape(R // 16, 16, C // 128, 2, 4, 16).transpose(0, 2, 3, 4, 1, 5)
    return np.ascontiguousarray(t).reshape(R, C)


def run_fprop(fp8, Xq, sX, Wq, sW, out_dtype=torch.bfloat16):
    C = fp8.block_gemm("fprop", dev(Xq), act_scales_dev(sX), dev(Wq), dev(sW), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("case", ["toy", "ragged", "lossless", "unit_scale", "fp32_out", "nan_scale"])
def test_fprop_small(gpu_lib, case):
    out = "bf16"
    if case == "toy":
        xb, wb = syn.toy_layer(0)
    elif case in ("ragged", "fp32_out", "nan_scale"):
        xb = syn.activation_with_outliers(333, 640, seed=21)
        wb = syn.gaussian((384, 640), seed=22, std=0.02)
    elif case == "lossless":
        xb, _ = syn.lossless_tiles(200, 384, seed=23, tile=(1, 128), k_range=(-6, 6))
        wb, _ = syn.lossless_tiles(256, 384, seed=24, tile=(128, 128), k_range=(-6, 6))
    else:
        xb = syn.activation_with_outliers(128, 512, seed=25)
        wb = syn.gaussian((256, 512), seed=26)
    Xq, sX = quant.quant_rows(xb)
    Wq, sW = quant.quant_weight(wb)
    if case == "unit_scale":
        sX = np.ones_like(sX)
        sW = np.ones_like(sW)
    if case == "nan_scale":
        sX = sX.copy()
        sX[7, 2] = np.nan
    R, T = og.fprop(Xq, sX, Wq, sW, with_magnitude=True)
    E = truncation_bound(Xq, sX, Wq, og.expand_block_scales(sW, Wq.shape[0]))
    if case == "fp32_out":
        C = run_fprop(gpu_lib, Xq, sX, Wq, sW, torch.float32)
        check_gemm(C.cpu().numpy(), R, T, Xq.shape[1], out="fp32", E=E, label=case)
    else:
        C = run_fprop(gpu_lib, Xq, sX, Wq, sW)
        check_gemm(bf16_bits(C), R, T, Xq.shape[1], out=out, E=E, label=case)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_many_tiles_per_workgroup_ragged(gpu_lib, out_dtype):
    """More tiles than CUs, so each persistent workgroup walks several (the
    next tile's loads issued before the current tile's stores), with ragged
    last rows and columns: full tiles take the staged epilogue, edge tiles the
    lane-by-lane stores.  Every output is checked against the oracle, and the
    operand-tiled run must match the row-major one bit for bit."""
    xb = syn.activation_with_outliers(4168, 256, seed=81)       # 33 row tiles, last 72 rows
    wb = syn.gaussian((2432, 256), seed=82, std=0.02)            # 9.5 column tiles of 256
    Xq, sX = quant.quant_rows(xb)
    Wq, sW = quant.quant_weight(wb)
    R, T = og.fprop(Xq, sX, Wq, sW, with_magnitude=True)
    E = truncation_bound(Xq, sX, Wq, og.expand_block_scales(sW, Wq.shape[0]))
    C = run_fprop(gpu_lib, Xq, sX, Wq, sW, out_dtype)
    if out_dtype == torch.float32:
        check_gemm(C.cpu().numpy(), R, T, 256, out="fp32", E=E, label="330 tiles fp32")
    else:
        check_gemm(bf16_bits(C), R, T, 256, E=E, label="330 tiles bf16")
    qt, st, _ = gpu_lib.quant_weight_128x128(dev(wb), tiled=True)
    Ct = gpu_lib.block_gemm("fprop_tiled", dev(Xq), act_scales_dev(sX), qt, st, out_dtype=out_dtype)
    torch.cuda.synchronize()
    view = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    assert torch.equal(C.view(view), Ct.view(view))


def test_fprop_full_size_sampled(gpu_lib, big_layer):
    """The configuration the bench times (operand-tiled weight codes,
    4096x18432x7168, persistent workgroups walking 9 tiles each, the next
    tile's loads overlapping the current tile's stores): one output row in
    every 128-row tile against the oracle, and a second launch byte-identical
    to the first."""
    Xq, sX, Wq, sW = big_layer
    A, sA, B, sB = dev(Xq), act_scales_dev(sX), dev(tiled_bytes(Wq)), dev(sW)
    C = gpu_lib.block_gemm("fprop_tiled", A, sA, B, sB)
    C2 = gpu_lib.block_gemm("fprop_tiled", A, sA, B, sB)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16)), "two launches differ"
    rows = rows_one_per_tile(4096, seed=3)
    R, T = og.fprop(Xq[rows], sX[rows], Wq, sW, with_magnitude=True)
    sWn = og.expand_block_scales(sW, 18432)
    stats = check_gemm(bf16_bits(C)[rows], R, T, 7168, label="fprop_tiled 4096x18432x7168",
                       E_at=lambda r, c: truncation_bound_at(Xq[rows], sX[rows], Wq, sWn, r, c))
    assert stats["n"] == rows.size * 18432


def test_tiled_bytes_reshape_matches_the_oracle_layout():
    from oracle import tiling
    q = np.random.default_rng(9).integers(0, 256, (48, 384), dtype=np.uint8)
    assert np.array_equal(tiled_bytes(q).ravel(), tiling.tile_codes(q))


def test_fprop_deterministic(gpu_lib):
    xb = syn.activation_with_outliers(512, 1024, seed=27)
    wb = syn.gaussian((512, 1024), seed=28, std=0.02)
    Xq, sX = quant.quant_rows(xb)
    Wq, sW = quant.quant_weight(wb)
    a = run_fprop(gpu_lib, Xq, sX, Wq, sW)
    b = run_fprop(gpu_lib, Xq, sX, Wq, sW)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def run_dgrad(fp8, dYq, s_dY, Wq, sW):
    C = fp8.block_gemm("dgrad", dev(dYq), act_scales_dev(s_dY), dev(Wq), dev(sW))
    torch.cuda.synchronize()
    return C


def test_dgrad_small_and_layout_identity(gpu_lib):
    dyb = syn.gaussian((200, 384), seed=31, std=1e-3)          # [tokens][d_out]
    wb = syn.gaussian((384, 256), seed=32, std=0.02)            # W [d_out][d_in]
    dYq, s_dY = quant.quant_rows(dyb)
    Wq, sW = quant.quant_weight(wb)
    R, T = og.dgrad(dYq, s_dY, Wq, sW, with_magnitude=True)
    E = truncation_bound(dYq, s_dY, np.ascontiguousarray(Wq.T), og.expand_block_scales(sW.T, 256))
    C = run_dgrad(gpu_lib, dYq, s_dY, Wq, sW)
    check_gemm(bf16_bits(C), R, T, 384, E=E, label="dgrad small")
    # same numbers as Fprop on the explicitly transposed weights
    F = run_fprop(gpu_lib, dYq, s_dY, np.ascontiguousarray(Wq.T), np.ascontiguousarray(sW.T))
    assert torch.equal(C.view(torch.int16), F.view(torch.int16))


def test_dgrad_full_size_sampled(gpu_lib, big_layer):
    _, _, Wq, sW = big_layer
    dyb = syn.gaussian((4096, 18432), seed=4, std=1e-3)
    dYq, s_dY = quant.quant_rows(dyb)
    del dyb
    C = run_dgrad(gpu_lib, dYq, s_dY, Wq, sW)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 4095], rng.choice(4096, 6, replace=False)]))
    R, T = og.dgrad(dYq[rows], s_dY[rows], Wq, sW, with_magnitude=True)
    Wt = np.ascontiguousarray(Wq.T)
    sWt = og.expand_block_scales(np.ascontiguousarray(sW.T), 7168)
    check_gemm(bf16_bits(C)[rows], R, T, 18432, label="dgrad (LDS) 4096x7168x18432",
               E_at=lambda r, c: truncation_bound_at(dYq[rows], s_dY[rows], Wt, sWt, r, c))


def run_dgrad_t(fp8, dYq, s_dY, Wq_t, sW):
    C = fp8.block_gemm("dgrad_t", dev(dYq), act_scales_dev(s_dY), dev(Wq_t), dev(sW))
    torch.cuda.synchronize()
    return C


def test_dgrad_t_small_with_gpu_transposed_codes(gpu_lib):
    """Dgrad from W_q^T: the weight quantizer's transposed codes feed the
    Fprop-shaped kernel with the forward scale table read transposed."""
    dyb = syn.gaussian((200, 384), seed=31, std=1e-3)          # [tokens][d_out]
    wb = syn.gaussian((384, 256), seed=32, std=0.02)            # W [d_out][d_in]
    dYq, s_dY = quant.quant_rows(dyb)
    Wq, sW = quant.quant_weight(wb)
    q, s, q_t = gpu_lib.quant_weight_128x128(dev(wb), transposed=True)
    torch.cuda.synchronize()
    assert np.array_equal(q_t.cpu().numpy(), np.ascontiguousarray(Wq.T))
    R, T = og.dgrad(dYq, s_dY, Wq, sW, with_magnitude=True)
    E = truncation_bound(dYq, s_dY, np.ascontiguousarray(Wq.T), og.expand_block_scales(sW.T, 256))
    C = gpu_lib.block_gemm("dgrad_t", dev(dYq), act_scales_dev(s_dY), q_t, s)
    torch.cuda.synchronize()
    check_gemm(bf16_bits(C), R, T, 384, E=E, label="dgrad_t small")
    # the same kernel as Fprop on the explicitly transposed weights and scales
    F = run_fprop(gpu_lib, dYq, s_dY, np.ascontiguousarray(Wq.T), np.ascontiguousarray(sW.T))
    assert torch.equal(C.view(torch.int16), F.view(torch.int16))


def test_dgrad_t_full_size_sampled(gpu_lib, big_layer):
    """The bench's Dgrad (operand-tiled W_q^T, 4096x7168x18432): one row per
    M tile against the oracle; two launches byte-identical."""
    _, _, Wq, sW = big_layer
    dyb = syn.gaussian((4096, 18432), seed=4, std=1e-3)
    dYq, s_dY = quant.quant_rows(dyb)
    del dyb
    Wt = np.ascontiguousarray(Wq.T)
    A, sA, B, sB = dev(dYq), act_scales_dev(s_dY), dev(tiled_bytes(Wt)), dev(sW)
    C = gpu_lib.block_gemm("dgrad_t_tiled", A, sA, B, sB)
    C2 = gpu_lib.block_gemm("dgrad_t_tiled", A, sA, B, sB)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16)), "two launches differ"
    rows = rows_one_per_tile(4096, seed=6)
    R, T = og.dgrad(dYq[rows], s_dY[rows], Wq, sW, with_magnitude=True)
    sWt = og.expand_block_scales(np.ascontiguousarray(sW.T), 7168)
    check_gemm(bf16_bits(C)[rows], R, T, 18432, label="dgrad_t_tiled 4096x7168x18432",
               E_at=lambda r, c: truncation_bound_at(dYq[rows], s_dY[rows], Wt, sWt, r, c))


def run_wgrad(fp8, dYt, s_dy, Xt, s_x, out_dtype=torch.float32):
    C = fp8.block_gemm("wgrad", dev(dYt), act_scales_dev(s_dy), dev(Xt), act_scales_dev(s_x),
                       out_dtype=out_dtype)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("out", ["fp32", "bf16"])
def test_wgrad_small(gpu_lib, out):
    dyb = syn.gaussian((256, 200), seed=41, std=1e-3)          # [tokens][d_out], ragged d_out
    xb = syn.activation_with_outliers(256, 136, seed=42)        # [tokens][d_in], ragged d_in
    dYt, s_dy = quant.quant_cols(dyb)
    Xt, s_x = quant.quant_cols(xb)
    R, T = og.wgrad(dYt, s_dy, Xt, s_x, with_magnitude=True)
    E = truncation_bound(dYt, s_dy, Xt, s_x)
    C = run_wgrad(gpu_lib, dYt, s_dy, Xt, s_x, torch.float32 if out == "fp32" else torch.bfloat16)
    y = C.cpu().numpy() if out == "fp32" else bf16_bits(C)
    check_gemm(y, R, T, 256, out=out, E=E, label=f"wgrad small {out}")


def test_wgrad_full_size_sampled(gpu_lib):
    """The bench's Wgrad (operand-tiled X_q^T, 18432x7168x4096, FP32 out):
    one row per M tile (144) against the oracle; two launches
    byte-identical."""
    dyb = syn.gaussian((4096, 18432), seed=4, std=1e-3)
    xb = syn.activation_with_outliers(4096, 7168, seed=0)
    dYt, s_dy = quant.quant_cols(dyb)
    del dyb
    Xt, s_x = quant.quant_cols(xb)
    del xb
    A, sA, B, sB = dev(dYt), act_scales_dev(s_dy), dev(tiled_bytes(Xt)), act_scales_dev(s_x)
    C = gpu_lib.block_gemm("wgrad_tiled", A, sA, B, sB, out_dtype=torch.float32)
    C2 = gpu_lib.block_gemm("wgrad_tiled", A, sA, B, sB, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int32), C2.view(torch.int32)), "two launches differ"
    rows = rows_one_per_tile(18432, seed=6)
    R, T = og.wgrad(dYt[rows], s_dy[rows], Xt, s_x, with_magnitude=True)
    check_gemm(C.cpu().numpy()[rows], R, T, 4096, out="fp32", label="wgrad_tiled 18432x7168x4096",
               E_at=lambda r, c: truncation_bound_at(dYt[rows], s_dy[rows], Xt, s_x, r, c))


def run_grouped(fp8, Xq, sX, offsets, Wq_e, sW_e):
    C = fp8.block_gemm_grouped(dev(offsets.astype(np.int32)), dev(Xq), act_scales_dev(sX),
                               dev(np.stack(Wq_e)), dev(np.stack(sW_e)))
    torch.cuda.synchronize()
    return C


def test_grouped_small_with_empty_and_tiny_groups(gpu_lib):
    counts = np.array([3, 0, 130, 1, 257, 0])
    off = syn.expert_offsets(counts)
    xb = syn.activation_with_outliers(int(counts.sum()), 384, seed=51)
    Xq, sX = quant.quant_rows(xb)
    ws = [quant.quant_weight(syn.gaussian((256, 384), seed=60 + e, std=0.02)) for e in range(6)]
    Wq_e, sW_e = [w[0] for w in ws], [w[1] for w in ws]
    R, T = og.grouped_fprop(Xq, sX, off, Wq_e, sW_e, with_magnitude=True)
    E = np.concatenate([truncation_bound(Xq[off[e]:off[e + 1]], sX[off[e]:off[e + 1]], Wq_e[e],
                                         og.expand_block_scales(sW_e[e], 256)) for e in range(6)])
    C = run_grouped(gpu_lib, Xq, sX, off, Wq_e, sW_e)
    check_gemm(bf16_bits(C), R, T, 384, E=E, label="grouped small")


@pytest.mark.parametrize("groups", [64, 80])
def test_grouped_many_groups(gpu_lib, groups):
    """Up to 64 groups the persistent kernel decodes tiles through a copy of
    the group table in LDS, beyond that through the offsets in device memory:
    64 and 80 groups (empty, one-row and multi-tile groups, K 256, N 256)
    against the oracle, row-major and operand-tiled weights bit-identical."""
    rng = np.random.default_rng(900 + groups)
    counts = rng.integers(0, 300, size=groups)
    counts[::7] = 0
    counts[3] = 1
    off = syn.expert_offsets(counts)
    K, N = 256, 256
    xb = syn.activation_with_outliers(int(counts.sum()), K, seed=71)
    Xq, sX = quant.quant_rows(xb)
    ws = [quant.quant_weight(syn.gaussian((N, K), seed=2000 + e, std=0.02)) for e in range(groups)]
    Wq_e, sW_e = [w[0] for w in ws], [w[1] for w in ws]
    R, T = og.grouped_fprop(Xq, sX, off, Wq_e, sW_e, with_magnitude=True)
    E = np.concatenate([truncation_bound(Xq[off[e]:off[e + 1]], sX[off[e]:off[e + 1]], Wq_e[e],
                                         og.expand_block_scales(sW_e[e], N)) for e in range(groups)])
    C = run_grouped(gpu_lib, Xq, sX, off, Wq_e, sW_e)
    offd = dev(off.astype(np.int32))
    Ct = gpu_lib.block_gemm_grouped(offd, dev(Xq), act_scales_dev(sX),
                                    dev(np.stack([tiled_bytes(w) for w in Wq_e])), dev(np.stack(sW_e)),
                                    tiled=True)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), Ct.view(torch.int16)), "tiled and row-major differ"
    check_gemm(bf16_bits(C), R, T, K, E=E, label=f"grouped {groups} groups")


def test_grouped_full_size_sampled(gpu_lib):
    """Config 5 as the bench times it (8 experts, 16384 tokens split by a
    seeded multinomial, N 2048, K 7168, operand-tiled expert weights): one row
    per M tile of every expert (its first and last row included) against the
    oracle, the tiled launch bit-identical to the row-major one, and two
    tiled launches byte-identical."""
    counts = syn.expert_counts(16384, 8, seed=0)
    off = syn.expert_offsets(counts)
    xb = syn.activation_with_outliers(16384, 7168, seed=0)
    Xq, sX = quant.quant_rows(xb)
    del xb
    ws = [quant.quant_weight(syn.gaussian((2048, 7168), seed=100 + e, std=0.02)) for e in range(8)]
    Wq_e, sW_e = [w[0] for w in ws], [w[1] for w in ws]
    offd, A, sA = dev(off.astype(np.int32)), dev(Xq), act_scales_dev(sX)
    S = dev(np.stack(sW_e))
    C_rm = gpu_lib.block_gemm_grouped(offd, A, sA, dev(np.stack(Wq_e)), S)
    Bt = dev(np.stack([tiled_bytes(w) for w in Wq_e]))
    C = gpu_lib.block_gemm_grouped(offd, A, sA, Bt, S, tiled=True)
    C2 = gpu_lib.block_gemm_grouped(offd, A, sA, Bt, S, tiled=True)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), C_rm.view(torch.int16)), "tiled and row-major differ"
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16)), "two launches differ"
    y = bf16_bits(C)
    for e in range(8):
        lo, hi = int(off[e]), int(off[e + 1])
        rows = lo + rows_one_per_tile(hi - lo, seed=7 + e)
        R, T = og.fprop(Xq[rows], sX[rows], Wq_e[e], sW_e[e], with_magnitude=True)
        sWn = og.expand_block_scales(sW_e[e], 2048)
        check_gemm(y[rows], R, T, 7168, label=f"grouped_tiled expert {e} ({hi - lo} rows)",
                   E_at=lambda r, c: truncation_bound_at(Xq[rows], sX[rows], Wq_e[e], sWn, r, c))


def test_grouped_malformed_offsets_stay_inside_the_rows(gpu_lib):
    """Offsets that break the contract (past total_M, decreasing, negative)
    are clamped on the device: C has guard rows beyond total_M that must keep
    their sentinel, the well-formed leading groups are still exact, and
    nothing faults.  Every access stays inside the allocations by
    construction: A, sA and C hold total_M (+ guard) rows."""
    total_M, N, K = 300, 256, 256
    xb = syn.activation_with_outliers(total_M, K, seed=121)
    Xq, sX = quant.quant_rows(xb)
    ws = [quant.quant_weight(syn.gaussian((N, K), seed=122 + e, std=0.02)) for e in range(5)]
    Wq_e, sW_e = [w[0] for w in ws], [w[1] for w in ws]
    B, S = dev(np.stack(Wq_e)), dev(np.stack(sW_e))
    guard = 64
    sentinel = 0x5A5A
    # (offsets, whether rows 0..99 stay group 0's alone after the clamp)
    for off, exact0 in (([0, 100, 5000, 150, 120, 300], True),
                        ([0, 100, 250, 2**31 - 1, 2**31 - 1, 2**31 - 1], True),
                        ([-50, 100, 200, 150, -7, 400], False)):
        offd = dev(np.asarray(off, np.int32))
        for tiled in (False, True):
            Cbuf = torch.full((total_M + guard, N), sentinel, dtype=torch.int16, device="cuda")
            Bx = dev(np.stack([tiled_bytes(w) for w in Wq_e])) if tiled else B
            gpu_lib.block_gemm_grouped(offd, dev(Xq), act_scales_dev(sX), Bx, S, tiled=tiled,
                                       out=Cbuf[:total_M].view(torch.bfloat16))
            torch.cuda.synchronize()
            assert torch.all(Cbuf[total_M:] == sentinel).item(), (off, tiled)
            if not exact0:
                continue
            R, T = og.fprop(Xq[:100], sX[:100], Wq_e[0], sW_e[0], with_magnitude=True)
            check_gemm(Cbuf[:100].cpu().numpy().view(np.uint16), R, T, K,
                       E=truncation_bound(Xq[:100], sX[:100], Wq_e[0], og.expand_block_scales(sW_e[0], N)),
                       label=f"grouped clamp {off[:4]} tiled={tiled}")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (5, 128, 256), (129, 128, 384)])
def test_degenerate_shapes(gpu_lib, M, N, K):
    """Edge shapes: a single token row; one 128-wide column block (half of a
    256-wide output tile, the other half past N); one K block (a pipeline
    round of four steps, three of them padding that folds with scale 0); a
    row tile holding one valid row after a full one.  BF16 out against the
    oracle; the operand-tiled weights bit-identical to the row-major ones."""
    xb = syn.activation_with_outliers(M, K, seed=1000 + M)
    wb = syn.gaussian((N, K), seed=2000 + N, std=0.02)
    Xq, sX = quant.quant_rows(xb)
    Wq, sW = quant.quant_weight(wb)
    R, T = og.fprop(Xq, sX, Wq, sW, with_magnitude=True)
    sWn = og.expand_block_scales(sW, N)
    C = run_fprop(gpu_lib, Xq, sX, Wq, sW)
    check_gemm(bf16_bits(C), R, T, K, label=f"degenerate {M}x{N}x{K}",
               E_at=lambda r, c: truncation_bound_at(Xq, sX, Wq, sWn, r, c))
    Ct = gpu_lib.block_gemm("fprop_tiled", dev(Xq), act_scales_dev(sX), dev(tiled_bytes(Wq)), dev(sW))
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), Ct.view(torch.int16))


def test_single_row_against_full_weights(gpu_lib, big_layer):
    """One token row (M = 1: one row tile with 127 rows past M) against the
    full 18432x7168 weights, every output element against the oracle, and
    equal to that row of the full 4096-row launch: a tile's rows do not
    interact."""
    Xq, sX, Wq, sW = big_layer
    B, sB = dev(tiled_bytes(Wq)), dev(sW)
    C1 = gpu_lib.block_gemm("fprop_tiled", dev(Xq[:1]), act_scales_dev(sX[:1]), B, sB)
    C = gpu_lib.block_gemm("fprop_tiled", dev(Xq), act_scales_dev(sX), B, sB)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C[:1].view(torch.int16)), "row 0 alone differs from row 0 of the layer"
    R, T = og.fprop(Xq[:1], sX[:1], Wq, sW, with_magnitude=True)
    sWn = og.expand_block_scales(sW, 18432)
    check_gemm(bf16_bits(C1), R, T, 7168, label="one row 1x18432x7168",
               E_at=lambda r, c: truncation_bound_at(Xq[:1], sX[:1], Wq, sWn, r, c))


@pytest.mark.parametrize("tiled", [False, True])
def test_grouped_single_group_equals_fprop(gpu_lib, tiled):
    """One group holding every row is a plain Fprop: the grouped launch must
    equal fp8_block_gemm bit for bit (the same tiles in the same order, the
    same split schedule).  4174 rows x N 2048 x K 1024 gives 264 tiles: more
    than one per persistent workgroup, a ragged last row tile and a split
    tail of 8 tiles; one row per M tile is also checked against the
    oracle."""
    M, N, K = 4174, 2048, 1024
    xb = syn.activation_with_outliers(M, K, seed=91)
    wb = syn.gaussian((N, K), seed=92, std=0.02)
    Xq, sX = quant.quant_rows(xb)
    Wq, sW = quant.quant_weight(wb)
    A, sA = dev(Xq), act_scales_dev(sX)
    B = dev(tiled_bytes(Wq)) if tiled else dev(Wq)
    C = gpu_lib.block_gemm("fprop_tiled" if tiled else "fprop", A, sA, B, dev(sW))
    off = dev(np.array([0, M], np.int32))
    Cg = gpu_lib.block_gemm_grouped(off, A, sA, B.reshape(1, N, K).contiguous(), dev(sW[None]), tiled=tiled)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), Cg.view(torch.int16)), "grouped (one group) and plain Fprop differ"
    rows = rows_one_per_tile(M, seed=93)
    R, T = og.fprop(Xq[rows], sX[rows], Wq, sW, with_magnitude=True)
    sWn = og.expand_block_scales(sW, N)
    check_gemm(bf16_bits(Cg)[rows], R, T, K, label=f"grouped one group {M}x{N}x{K}",
               E_at=lambda r, c: truncation_bound_at(Xq[rows], sX[rows], Wq, sWn, r, c))


# ---------------------------------------------------------------------------
# Operand-tiled weight codes: the quantizer's tiled bytes against the
# oracle's layout, and every tiled GEMM bit-identical to its row-major twin.
# ---------------------------------------------------------------------------
def test_tiled_weight_codes_match_the_layout(gpu_lib):
    from oracle import tiling
    wb = syn.gaussian((384, 640), seed=71, std=0.02)
    Wq, sW = quant.quant_weight(wb)
    q, s, q_t = gpu_lib.quant_weight_128x128(dev(wb), transposed=True, tiled=True)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy().ravel(), tiling.tile_codes(Wq))
    assert np.array_equal(q_t.cpu().numpy().ravel(), tiling.tile_codes(np.ascontiguousarray(Wq.T)))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), sW.view(np.uint32))


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_tiled_fprop_and_dgrad_t_bit_identical(gpu_lib, out_dtype):
    xb = syn.activation_with_outliers(300, 640, seed=72)      # ragged M
    wb = syn.gaussian((384, 640), seed=73, std=0.02)            # W [N][K]
    x = dev(xb)
    xq, xs, _ = gpu_lib.quant_act_1x128(x, "row")
    q, s, q_t = gpu_lib.quant_weight_128x128(dev(wb), transposed=True)
    qt, st, qt_t = gpu_lib.quant_weight_128x128(dev(wb), transposed=True, tiled=True)
    a = gpu_lib.block_gemm("fprop", xq, xs, q, s, out_dtype=out_dtype)
    b = gpu_lib.block_gemm("fprop_tiled", xq, xs, qt, st, out_dtype=out_dtype)
    dyb = syn.gaussian((300, 384), seed=74, std=1e-3)            # dY [tokens][N]
    dq, ds, _ = gpu_lib.quant_act_1x128(dev(dyb), "row")
    c = gpu_lib.block_gemm("dgrad_t", dq, ds, q_t, s, out_dtype=out_dtype)
    d = gpu_lib.block_gemm("dgrad_t_tiled", dq, ds, qt_t, st, out_dtype=out_dtype)
    torch.cuda.synchronize()
    view = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    assert torch.equal(a.view(view), b.view(view))
    assert torch.equal(c.view(view), d.view(view))


def test_tiled_full_size_bit_identical(gpu_lib):
    x = dev(syn.activation_with_outliers(4096, 7168, seed=0))
    w = dev(syn.gaussian((18432, 7168), seed=1, std=0.02))
    xq, xs, _ = gpu_lib.quant_act_1x128(x, "row")
    q, s, q_t = gpu_lib.quant_weight_128x128(w, transposed=True)
    a = gpu_lib.block_gemm("fprop", xq, xs, q, s)
    del q
    qt, st, qt_t = gpu_lib.quant_weight_128x128(w, transposed=True, tiled=True)
    b = gpu_lib.block_gemm("fprop_tiled", xq, xs, qt, st)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    del a, b, qt
    dq, ds, _ = gpu_lib.quant_act_1x128(dev(syn.gaussian((4096, 18432), seed=4, std=1e-3)), "row")
    c = gpu_lib.block_gemm("dgrad_t", dq, ds, q_t, s)
    d = gpu_lib.block_gemm("dgrad_t_tiled", dq, ds, qt_t, st)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), d.view(torch.int16))


def test_tiled_grouped_bit_identical(gpu_lib):
    counts = np.array([3, 0, 130, 1, 257, 0, 600, 64])
    off = dev(syn.expert_offsets(counts).astype(np.int32))
    x = dev(syn.activation_with_outliers(int(counts.sum()), 1024, seed=75))
    xq, xs, _ = gpu_lib.quant_act_1x128(x, "row")
    ws = [gpu_lib.quant_weight_128x128(dev(syn.gaussian((256, 1024), seed=80 + e, std=0.02)))
          for e in range(8)]
    wt = [gpu_lib.quant_weight_128x128(dev(syn.gaussian((256, 1024), seed=80 + e, std=0.02)), tiled=True)
          for e in range(8)]
    B = torch.stack([w[0] for w in ws]).contiguous()
    Bt = torch.stack([w[0] for w in wt]).contiguous()
    S = torch.stack([w[1] for w in ws]).contiguous()
    for out_dtype, view in ((torch.bfloat16, torch.int16), (torch.float32, torch.int32)):
        a = gpu_lib.block_gemm_grouped(off, xq, xs, B, S, out_dtype=out_dtype)
        b = gpu_lib.block_gemm_grouped(off, xq, xs, Bt, S, tiled=True, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(a.view(view), b.view(view))


def test_tiled_column_codes_and_wgrad(gpu_lib):
    """128x1 column codes written operand-tiled (column quantizer and dual
    pass) match the oracle's layout, and Wgrad reading them is bit-identical
    to Wgrad on the row-major codes."""
    from oracle import tiling
    xb = syn.activation_with_outliers(384, 640, seed=91)        # X [tokens][d_in]
    dyb = syn.gaussian((384, 256), seed=92, std=1e-3)            # dY [tokens][d_out]
    x, dy = dev(xb), dev(dyb)
    qx, sx, _ = gpu_lib.quant_act_1x128(x, "col")
    qx_t, sx_t, _ = gpu_lib.quant_act_1x128(x, "col_tiled")
    qo, _ = quant.quant_cols(xb)
    assert np.array_equal(qx_t.cpu().numpy().ravel(), tiling.tile_codes(qo))
    assert torch.equal(sx, sx_t)
    r0, s0, c0, t0 = gpu_lib.quant_act_dual(x)
    r1, s1, c1, t1 = gpu_lib.quant_act_dual(x, tiled=True)
    assert torch.equal(r0, r1) and torch.equal(s0, s1) and torch.equal(t0, t1)
    assert torch.equal(c1, qx_t)
    qd, sd, _ = gpu_lib.quant_act_1x128(dy, "col")
    for out_dtype, view in ((torch.float32, torch.int32), (torch.bfloat16, torch.int16)):
        a = gpu_lib.block_gemm("wgrad", qd, sd, qx, sx, out_dtype=out_dtype)
        b = gpu_lib.block_gemm("wgrad_tiled", qd, sd, qx_t, sx_t, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(a.view(view), b.view(view))


def test_tiled_wgrad_full_size_bit_identical(gpu_lib):
    x = dev(syn.activation_with_outliers(4096, 7168, seed=0))
    dy = dev(syn.gaussian((4096, 18432), seed=4, std=1e-3))
    _, _, qd, sd = gpu_lib.quant_act_dual(dy)
    _, _, qx, sx = gpu_lib.quant_act_dual(x)
    _, _, qx_t, sx_t = gpu_lib.quant_act_dual(x, tiled=True)
    a = gpu_lib.block_gemm("wgrad", qd, sd, qx, sx, out_dtype=torch.float32)
    b = gpu_lib.block_gemm("wgrad_tiled", qd, sd, qx_t, sx_t, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("mode", ["plain", "scaled", "fold"])
def test_probe_mfma_counts_its_work(gpu_lib, mode):
    """The rate probe runs 8 * iters MFMAs per wave in every mode: with every
    code 1.0 each of a lane's 4 outputs per chain gains 128 per MFMA (the
    fold multiplies by 1.0), so its checksum is 8 * 4 * 128 * iters; with
    zero codes it is 0.  Odd and even iteration counts (the fold mode runs
    rounds in pairs)."""
    ones = torch.full((4096,), 0x38, dtype=torch.uint8, device="cuda")
    out = gpu_lib.probe_mfma(ones, 3, 5, mode)
    out6 = gpu_lib.probe_mfma(ones, 2, 6, mode)
    zero = gpu_lib.probe_mfma(torch.zeros(4096, dtype=torch.uint8, device="cuda"), 2, 7, mode)
    torch.cuda.synchronize()
    assert torch.all(out == 8 * 4 * 128 * 5).item()
    assert torch.all(out6 == 8 * 4 * 128 * 6).item()
    assert torch.all(zero == 0).item()
