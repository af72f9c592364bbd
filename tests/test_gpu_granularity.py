"""GPU parity of the tile-size / percentile-clipping quantizer against the
oracle (bit-exact codes, scales and saturation counts), and the pages' two
granularity labs measured on it: error against tile size with the scale
metadata it costs, and percentile clipping on the outlier recipe.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import granularity as gr
from oracle import quant
from test_gpu_quant import adversarial_rows

pytestmark = pytest.mark.gpu


def dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.int16) if t.dtype == torch.uint16 else t).cuda()


def run(fp8, x, tile, rank):
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    q, s = fp8.quant_act_tiles(dev(x), tile, rank, sat_count=sat)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()[:, :x.shape[0]].T, int(sat.item())


def check(fp8, x, tile, rank, label=""):
    q, s, sat = run(fp8, x, tile, rank)
    q0, s0, sat0 = gr.quant_rows_tiles(x, tile, rank)
    assert np.array_equal(s.view(np.uint32), s0.view(np.uint32)), f"{label} T={tile} r={rank}: scales"
    bad = np.argwhere(q != q0)
    assert bad.size == 0, f"{label} T={tile} r={rank}: {len(bad)} codes differ, e.g. {bad[:3].tolist()}"
    assert sat == sat0, f"{label} T={tile} r={rank}: saturation {sat} vs {sat0}"
    return q, s, sat


@pytest.mark.parametrize("tile", gr.TILES)
@pytest.mark.parametrize("rank", [1, 2, 5, 8])
def test_tiles_outliers(gpu_lib, tile, rank):
    check(gpu_lib, syn.activation_with_outliers(37, 2048, seed=tile + rank), tile, rank, "outliers")


@pytest.mark.parametrize("tile", [32, 64, 128, 256])
@pytest.mark.parametrize("rank", [1, 3])
def test_tiles_adversarial(gpu_lib, tile, rank):
    check(gpu_lib, adversarial_rows(), tile, rank, "adversarial")


def test_tiles_lossless(gpu_lib):
    for tile in gr.TILES:
        x, k = syn.lossless_tiles(9, 3072, seed=tile, tile=(1, tile))
        _, s, _ = check(gpu_lib, x, tile, 1, "lossless")
        assert np.array_equal(s, np.exp2(k).astype(np.float32))


def test_tile_128_rank_1_is_the_row_quantizer(gpu_lib):
    x = dev(syn.activation_with_outliers(200, 1152, seed=9))
    q, s = gpu_lib.quant_act_tiles(x, 128, 1)
    q0, s0, _ = gpu_lib.quant_act_1x128(x, "row")
    torch.cuda.synchronize()
    assert torch.equal(q, q0)
    assert torch.equal(s[:, :200].view(torch.int32), s0[:, :200].view(torch.int32))


def test_tiles_full_size(gpu_lib):
    x = syn.activation_with_outliers(2048, 7168, seed=0)
    for tile, rank in ((32, 1), (1024, 2), (128, 4)):
        check(gpu_lib, x, tile, rank, "full")


def test_granularity_study(gpu_lib):
    """Error against tile size (online rule) and percentile clipping (T = 128)
    on X 1024x7168 with 16 outlier channels; errors from the GPU codes.

    Measured: the mean error falls only from 2.19e-2 (T = 1024) to 2.00e-2
    (T = 32) while the scale metadata grows from 0.4% to 12.5% of the code
    bytes; clipping at the 2nd largest value erases 61% of the outliers'
    magnitude and leaves the other values slightly worse."""
    M, K = 1024, 7168
    x = syn.activation_with_outliers(M, K, seed=0)
    xf = quant.bf16_to_f32(x).astype(np.float64)
    lines = []
    errs = {}
    for tile in gr.TILES:
        q, s, sat = check(gpu_lib, x, tile, 1, "study")
        d = np.abs(gr.dequant_tiles(q, s, tile) - xf)
        errs[tile] = np.mean(d) / np.mean(np.abs(xf))
        lines.append(f"T={tile:5d} rank 1  rel mean abs err {errs[tile]:.4e}  max abs err {d.max():.3e}  "
                     f"scale bytes/value {gr.metadata_bytes_per_value(tile):.5f} "
                     f"({100 * gr.metadata_bytes_per_value(tile):.2f}% of the codes)")
    vals = [errs[t] for t in gr.TILES]
    assert all(a < b for a, b in zip(vals, vals[1:]))
    # outlier cells are set to +-20; the N(0, 1) values never reach 16
    outl = np.abs(xf) >= 16
    e_out, e_rest, sats = {}, {}, {}
    for rank in (1, 2, 4, 8):
        q, s, sat = check(gpu_lib, x, 128, rank, "study")
        d = np.abs(gr.dequant_tiles(q, s, 128) - xf)
        e_out[rank] = np.mean(d[outl]) / np.mean(np.abs(xf[outl]))
        e_rest[rank] = np.mean(d[~outl]) / np.mean(np.abs(xf[~outl]))
        sats[rank] = sat
        lines.append(f"T=  128 rank {rank}  saturated {sat:7d}  rel err on outlier cells {e_out[rank]:.4e}  "
                     f"on the other values {e_rest[rank]:.4e}")
    print("\n" + "\n".join(lines))
    # Measured: the outliers come back exactly under the max rule and are
    # erased by clipping; the other values gain nothing, because E4M3 is a
    # floating-point code whose relative spacing does not depend on the scale
    # (only values pushed into its subnormal range would gain), while the
    # clipped Gaussian tail adds error.
    assert e_out[1] < 1e-6 and e_out[2] > 0.3
    assert e_out[1] < e_out[2] < e_out[4] <= e_out[8]
    assert all(e_rest[r] >= e_rest[1] for r in (2, 4, 8))
    assert sats[1] == 0 and sats[2] < sats[4] < sats[8]
