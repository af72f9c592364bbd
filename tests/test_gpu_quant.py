"""GPU parity of the quantizers against the oracle: bit-exact codes and scales.

Inputs are the seeded synthetic workloads (and adversarial tiles); the
expected values come only from ``oracle``.  Full-size cases run the kernel on
the whole tensor and compare a seeded sample of rows/columns/blocks exactly.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import e4m3, quant

pytestmark = pytest.mark.gpu


def dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.cuda()


def host(t):
    return t.cpu().numpy()


def scale_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_rows_match(fp8, x_bits, rows_idx=None, ldx_pad=0, label=""):
    M, K = x_bits.shape
    if ldx_pad:
        buf = np.zeros((M, K + ldx_pad), np.uint16)
        buf[:, :K] = x_bits
        xt = dev(buf)[:, :K]
    else:
        xt = dev(x_bits)
    q, s, amax = fp8.quant_act_1x128(xt, "row", return_amax=True)
    torch.cuda.synchronize()
    q, s, amax = host(q), host(s)[:, :M].T, host(amax)[:, :M].T
    sel = np.arange(M) if rows_idx is None else rows_idx
    q_o, s_o = quant.quant_rows(x_bits[sel])
    assert np.array_equal(q[sel], q_o), f"{label}: codes differ at {np.argwhere(q[sel] != q_o)[:5]}"
    assert np.array_equal(scale_bits(s[sel]), scale_bits(s_o)), f"{label}: scales differ"
    x = quant.bf16_to_f32(x_bits[sel]).reshape(len(sel), K // 128, 128)
    amax_o = np.max(np.abs(x), axis=-1)
    nan = np.isnan(amax_o)
    assert np.array_equal(np.isnan(amax[sel]), nan)
    assert np.array_equal(scale_bits(amax[sel])[~nan], scale_bits(amax_o)[~nan])


def adversarial_rows():
    """Tiles that exercise every special case of the rule, one per row."""
    rng = np.random.default_rng(123)
    rows = []

    def add(v):
        rows.append(syn.f32_to_bf16_bits(np.asarray(v, np.float32)))

    add(np.zeros(256))
    z = np.zeros(256, np.float32); z[::3] = -0.0; add(z)
    add(np.full(256, 3.0))                                    # constant tile: every code 0x7E
    add(np.full(256, -1e-30))                                 # tiny: floor scale
    sub = np.zeros(256, np.float32); sub[::7] = 2.0 ** -130; sub[1::7] = -(2.0 ** -133); add(sub)
    one = rng.standard_normal(256).astype(np.float32); one[5] = 20.0; one[200] = -300.0; add(one)
    big = rng.standard_normal(256).astype(np.float32) * 1e37; big[0] = 3.38e38; add(big)
    nan = rng.standard_normal(256).astype(np.float32); nan[17] = np.nan; add(nan)
    inf = rng.standard_normal(256).astype(np.float32); inf[3] = np.inf; inf[130] = -np.inf; add(inf)
    both = rng.standard_normal(256).astype(np.float32); both[9] = np.inf; both[10] = np.nan; add(both)
    # exact E4M3 midpoints after scaling: tile max 448 so s = 1
    mids = np.concatenate([e4m3.MIDPOINTS, -e4m3.MIDPOINTS[:2]]).astype(np.float32)
    mid = np.zeros(256, np.float32); mid[:mids.size] = mids; mid[255] = 448.0; add(mid)
    ramp = np.linspace(-1, 1, 256).astype(np.float32); add(ramp)
    bits = np.stack(rows)
    return bits


@pytest.mark.parametrize("case", ["toy", "ragged", "adversarial", "lossless", "padded_ld"])
def test_quant_rows_small(gpu_lib, case):
    if case == "toy":
        x, _ = syn.toy_layer(0)
        assert_rows_match(gpu_lib, x, label=case)
    elif case == "ragged":
        x = syn.activation_with_outliers(333, 1152, seed=4)
        assert_rows_match(gpu_lib, x, label=case)
    elif case == "adversarial":
        assert_rows_match(gpu_lib, adversarial_rows(), label=case)
    elif case == "lossless":
        x, _ = syn.lossless_tiles(130, 640, seed=5, tile=(1, 128))
        assert_rows_match(gpu_lib, x, label=case)
    else:
        x = syn.activation_with_outliers(70, 384, seed=6)
        assert_rows_match(gpu_lib, x, ldx_pad=64, label=case)


def test_quant_rows_full_size_sampled(gpu_lib):
    M, K = 8192, 7168
    x = syn.activation_with_outliers(M, K, seed=0)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 1, M - 1], rng.choice(M, 189, replace=False)]))
    assert_rows_match(gpu_lib, x, rows_idx=rows, label="8192x7168")


def test_quant_rows_deterministic(gpu_lib):
    x = dev(syn.activation_with_outliers(1024, 2048, seed=7))
    a = gpu_lib.quant_act_1x128(x)
    b = gpu_lib.quant_act_1x128(x)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def assert_cols_match(fp8, x_bits, cols_idx=None, label=""):
    M, C = x_bits.shape
    q, s, amax = fp8.quant_act_1x128(dev(x_bits), "col", return_amax=True)
    torch.cuda.synchronize()
    q, s = host(q), host(s)[:, :C].T                      # q [C][M], s [C][M/128]
    sel = np.arange(C) if cols_idx is None else cols_idx
    q_o, s_o = quant.quant_cols(x_bits[:, sel])
    assert np.array_equal(q[sel], q_o), f"{label}: codes differ"
    assert np.array_equal(scale_bits(s[sel]), scale_bits(s_o)), f"{label}: scales differ"


@pytest.mark.parametrize("case", ["gauss", "ragged_cols", "adversarial_t", "lossless"])
def test_quant_cols_small(gpu_lib, case):
    if case == "gauss":
        x = syn.gaussian((256, 384), seed=8, std=1e-3)
    elif case == "ragged_cols":
        x = syn.activation_with_outliers(384, 200, seed=9)
    elif case == "adversarial_t":
        a = adversarial_rows()                          # [12][256] -> columns of a [256][12+4]
        x = np.zeros((256, 16), np.uint16)
        x[:, :a.shape[0]] = a.T
    else:
        x, _ = syn.lossless_tiles(256, 136, seed=10, tile=(128, 1))
    assert_cols_match(gpu_lib, x, label=case)


def test_quant_cols_equals_rows_of_transpose(gpu_lib):
    x = syn.activation_with_outliers(512, 384, seed=11)
    qc, sc, _ = gpu_lib.quant_act_1x128(dev(x), "col")
    qr, sr, _ = gpu_lib.quant_act_1x128(dev(np.ascontiguousarray(x.T)), "row")
    torch.cuda.synchronize()
    assert torch.equal(qc, qr)
    assert torch.equal(sc[:, :384], sr[:, :384])


def test_quant_cols_full_size_sampled(gpu_lib):
    M, C = 4096, 18432
    x = syn.gaussian((M, C), seed=1, std=1e-3)
    rng = np.random.default_rng(1)
    cols = np.unique(np.concatenate([[0, C - 1], rng.choice(C, 126, replace=False)]))
    assert_cols_match(gpu_lib, x, cols_idx=cols, label="dY col 4096x18432")


def assert_dual_match(fp8, x_bits, label=""):
    """fp8_quant_act_dual = the oracle's row and column quantizations, bit for bit,
    and = the two separate GPU quantizations."""
    M, C = x_bits.shape
    xt = dev(x_bits)
    q_row, s_row, q_col, s_col = fp8.quant_act_dual(xt)
    qr, sr, _ = fp8.quant_act_1x128(xt, "row")
    qc, sc, _ = fp8.quant_act_1x128(xt, "col")
    torch.cuda.synchronize()
    assert torch.equal(q_row, qr) and torch.equal(q_col, qc), f"{label}: codes differ from separate passes"
    assert torch.equal(s_row[:, :M].view(torch.int32), sr[:, :M].view(torch.int32)), label
    assert torch.equal(s_col[:, :C].view(torch.int32), sc[:, :C].view(torch.int32)), label
    q_o, s_o = quant.quant_rows(x_bits)
    assert np.array_equal(host(q_row), q_o), f"{label}: row codes differ from the oracle"
    assert np.array_equal(scale_bits(host(s_row)[:, :M].T), scale_bits(s_o)), f"{label}: row scales"
    qc_o, sc_o = quant.quant_cols(x_bits)
    assert np.array_equal(host(q_col), qc_o), f"{label}: column codes differ from the oracle"
    assert np.array_equal(scale_bits(host(s_col)[:, :C].T), scale_bits(sc_o)), f"{label}: column scales"


@pytest.mark.parametrize("case", ["gauss", "outliers", "adversarial", "lossless_rows", "lossless_cols"])
def test_quant_dual_small(gpu_lib, case):
    if case == "gauss":
        x = syn.gaussian((256, 384), seed=12, std=1e-3)
    elif case == "outliers":
        x = syn.activation_with_outliers(384, 256, seed=13)
    elif case == "adversarial":
        # special-value tiles both along rows and, transposed, along columns
        a = adversarial_rows()                          # [12][256]
        x = np.zeros((256, 256), np.uint16)
        x[:a.shape[0], :] = a
        x[:, 128:128 + a.shape[0]] = a.T
    elif case == "lossless_rows":
        x, _ = syn.lossless_tiles(256, 256, seed=14, tile=(1, 128))
    else:
        x, _ = syn.lossless_tiles(256, 256, seed=15, tile=(128, 1))
    assert_dual_match(gpu_lib, x, label=case)


@pytest.mark.parametrize("M,K", [(1, 128), (1, 7168), (3, 256), (130, 128)])
def test_quant_rows_degenerate(gpu_lib, M, K):
    """One and a few rows, one tile wide and a layer wide, and a row count
    just past a multiple of 128: codes, scales and amax bit-exact."""
    x = syn.activation_with_outliers(M, K, seed=500 + M + K)
    assert_rows_match(gpu_lib, x, label=f"rows {M}x{K}")


@pytest.mark.parametrize("M,C", [(128, 8), (128, 128), (128, 7168)])
def test_quant_cols_and_dual_degenerate(gpu_lib, M, C):
    """One 128-token block: eight columns (the narrowest 16-byte row), one
    column block, and a layer wide; the dual pass where C is whole blocks."""
    x = syn.gaussian((M, C), seed=600 + C, std=1e-3)
    assert_cols_match(gpu_lib, x, label=f"cols {M}x{C}")
    if C % 128 == 0:
        assert_dual_match(gpu_lib, x, label=f"dual {M}x{C}")


def test_quant_into_caller_buffers(gpu_lib):
    """The binding's caller buffers (codes, and scales with a padded row
    stride) receive exactly what the allocating call returns."""
    x = dev(syn.activation_with_outliers(300, 640, seed=700))
    q0, s0, _ = gpu_lib.quant_act_1x128(x, "row")
    q = torch.full((300, 640), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((5, 320), -1.0, dtype=torch.float32, device="cuda")
    q1, s1, _ = gpu_lib.quant_act_1x128(x, "row", out=q, scales_out=s)
    torch.cuda.synchronize()
    assert q1.data_ptr() == q.data_ptr() and s1.data_ptr() == s.data_ptr()
    assert torch.equal(q, q0)
    assert torch.equal(s[:, :300].view(torch.int32), s0[:, :300].view(torch.int32))
    assert bool((s[:, 300:] == -1.0).all()), "scale padding columns written"
    with pytest.raises(ValueError):
        gpu_lib.quant_act_1x128(x, "row", out=torch.empty((300, 512), dtype=torch.uint8, device="cuda"))


def test_quant_dual_full_size(gpu_lib):
    """dY 4096x18432: both orientations equal the separate passes everywhere
    (compared on the GPU) and the oracle on a sample of rows and columns."""
    M, C = 4096, 18432
    x = syn.gaussian((M, C), seed=4, std=1e-3)
    xt = dev(x)
    q_row, s_row, q_col, s_col = gpu_lib.quant_act_dual(xt)
    qr, sr, _ = gpu_lib.quant_act_1x128(xt, "row")
    qc, sc, _ = gpu_lib.quant_act_1x128(xt, "col")
    torch.cuda.synchronize()
    assert torch.equal(q_row, qr) and torch.equal(q_col, qc)
    assert torch.equal(s_row[:, :M].view(torch.int32), sr[:, :M].view(torch.int32))
    assert torch.equal(s_col[:, :C].view(torch.int32), sc[:, :C].view(torch.int32))
    rng = np.random.default_rng(16)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 30, replace=False)]))
    q_o, s_o = quant.quant_rows(x[rows])
    assert np.array_equal(host(q_row)[rows], q_o)
    assert np.array_equal(scale_bits(host(s_row)[:, rows].T), scale_bits(s_o))
    cols = np.unique(np.concatenate([[0, C - 1], rng.choice(C, 30, replace=False)]))
    qc_o, sc_o = quant.quant_cols(x[:, cols])
    assert np.array_equal(host(q_col)[cols], qc_o)
    assert np.array_equal(scale_bits(host(s_col)[:, cols].T), scale_bits(sc_o))


def assert_weight_match(fp8, w_bits, blocks=None, label=""):
    N, K = w_bits.shape
    q, s, q_t = fp8.quant_weight_128x128(dev(w_bits), transposed=True)
    torch.cuda.synchronize()
    q, s, q_t = host(q), host(s), host(q_t)
    assert np.array_equal(q_t, q.T), f"{label}: transposed copy differs"
    if blocks is None:
        q_o, s_o = quant.quant_weight(w_bits)
        assert np.array_equal(q, q_o), f"{label}: codes differ"
        assert np.array_equal(scale_bits(s), scale_bits(s_o)), f"{label}: scales differ"
    else:
        for bi, bj in blocks:
            blk = w_bits[128 * bi:128 * (bi + 1), 128 * bj:128 * (bj + 1)]
            q_o, s_o = quant.quant_weight(blk)
            assert np.array_equal(q[128 * bi:128 * (bi + 1), 128 * bj:128 * (bj + 1)], q_o), label
            assert scale_bits(s[bi, bj]) == scale_bits(s_o[0, 0]), label


def test_quant_weight_small(gpu_lib):
    assert_weight_match(gpu_lib, syn.gaussian((384, 256), seed=12, std=0.02), label="gauss")
    _, w = syn.toy_layer(0)
    assert_weight_match(gpu_lib, w, label="toy")
    lw, _ = syn.lossless_tiles(256, 384, seed=13, tile=(128, 128))
    assert_weight_match(gpu_lib, lw, label="lossless")
    adv = np.zeros((128, 256), np.uint16)
    a = adversarial_rows()
    adv[:a.shape[0], :] = a
    adv[:, 128:] = 0                                   # second block all zero -> floor scale
    assert_weight_match(gpu_lib, adv, label="adversarial")


def test_quant_weight_full_size_sampled(gpu_lib):
    w = syn.gaussian((18432, 7168), seed=2, std=0.02)
    rng = np.random.default_rng(2)
    blocks = [(0, 0), (143, 55)] + [(int(rng.integers(144)), int(rng.integers(56))) for _ in range(14)]
    assert_weight_match(gpu_lib, w, blocks=blocks, label="W 18432x7168")


def _e4m3_thresholds():
    """Smallest non-negative fp32 bit pattern reaching each code 1..126 (oracle)."""
    thr = []
    for c in range(1, 127):
        lo, hi = 0, 0x7F800000
        while lo < hi:
            mid = (lo + hi) // 2
            if e4m3.encode(np.uint32(mid).view(np.float32)) >= c:
                hi = mid
            else:
                lo = mid + 1
        thr.append(lo)
        # pin: the oracle code changes exactly there
        assert e4m3.encode(np.uint32(lo).view(np.float32)) == c
        assert e4m3.encode(np.uint32(lo - 1).view(np.float32)) == c - 1
    return np.array(thr, dtype=np.int64)


def test_cast_exhaustive_all_fp32(gpu_lib):
    """Every one of the 2**32 FP32 bit patterns through the E4M3 cast."""
    thr = torch.from_numpy(_e4m3_thresholds()).cuda()
    chunk = 1 << 28
    for start in range(0, 1 << 31, chunk):
        bits = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda")
        x = bits.to(torch.int32).view(torch.float32)
        want = torch.bucketize(bits, thr, right=True).to(torch.uint8)
        want[bits > 0x7F800000] = 0x7F
        got = gpu_lib.cast_e4m3(x)
        assert torch.equal(got, want), f"positive patterns from {start:#x}"
        neg = (bits | 0x80000000).to(torch.int64)
        xn = (neg - (1 << 32)).to(torch.int32).view(torch.float32)
        wantn = want | 0x80
        wantn[bits > 0x7F800000] = 0x7F
        gotn = gpu_lib.cast_e4m3(xn)
        assert torch.equal(gotn, wantn), f"negative patterns from {start:#x}"
        del bits, x, want, got, neg, xn, wantn, gotn
    torch.cuda.synchronize()


def test_online_reciprocal_exact_on_every_online_scale(gpu_lib):
    """The quantizers take r = fl32(1/s) of an online scale from the hardware
    reciprocal estimate refined by one FMA Newton step.  The division
    shortcut's exhaustive host check assumes r is the IEEE reciprocal, so
    this checks exactly that on every scale the online rule can produce:
    s = max(fl32(a / 448), fl32(1e-12)) for every finite non-negative BF16 a
    (the reference reciprocal is numpy's correctly rounded float32 division)."""
    a = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    floor = np.array([0x2B8CBCCC], np.uint32).view(np.float32)[0]
    s = np.unique(np.maximum(a / np.float32(448.0), floor)).astype(np.float32)
    want = (np.float32(1.0) / s).astype(np.float32)
    got = gpu_lib.probe_recip_online(torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, [(float(s[i]), float(got[i]), float(want[i])) for i in bad[:5]]
