"""Worked examples and scale-policy invariants (CPU only).

Each test pins the oracle to a statement the pages make (inputs from
tests/golden/page_constants.json) or to arithmetic that follows from it.
"""
import json
import os

import numpy as np

from oracle import e4m3, examples, policies, quant
import synthetic as syn

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_two_tile_worked_example():
    r = examples.two_tiles(seed=0)
    g = GOLDEN["two_tile_example"]
    tiles = r["tiles"]
    assert tiles[1, 0] == g["outlier"] and abs(float(np.median(tiles[0])) - g["center"]) < 0.01
    # the outlier tile's own scale equals the global scale bit for bit ...
    assert r["s_local"][1].view(np.uint32) == r["s_global"].view(np.uint32)
    assert np.array_equal(r["q_global"][1], r["q_local"][1])
    # ... so local scaling changes only the quiet tile, and improves it
    assert r["err_local"][1] == r["err_global"][1]
    assert r["err_local"][0] < r["err_global"][0]
    # under the global scale the quiet tile lands in [1, 4): E4M3 spacing at most 0.25
    scaled = tiles[0] / r["s_global"]
    assert np.all((scaled >= 1) & (scaled < 4))
    assert np.all(r["abs_err_global"][0] <= 0.125 * float(r["s_global"]) * (1 + 2.0 ** -19))
    # scale bytes per activation value
    assert r["scale_bytes_per_value_local"] == GOLDEN["scale_bytes_per_value_1x128"]["value"]
    assert r["scale_bytes_per_value_global"] == 4 / 256


def test_fine_grained_gemm_error_below_per_tensor():
    g = GOLDEN["gemm_error_example"]
    assert (g["tokens"], g["in_channels"], g["out_channels"]) == (64, 512, 1024)
    r = examples.per_tensor_vs_fine()
    assert r["err_fine"] < r["err_per_tensor"]
    assert 0 < r["err_fine"] < 0.05


def test_outlier_shrink_arithmetic():
    g = GOLDEN["outlier_shrink_example"]
    # the page's figures are the small values divided by the outlier (max mapped to 1)
    got = [round(v / g["outlier"], 4) for v in g["small"]]
    assert got == g["page_scaled"]
    # under the max -> 448 rule the same tile keeps both small values normal in E4M3
    vals = np.zeros(128, np.float32)
    vals[0], vals[1], vals[2] = g["outlier"], g["small"][0], g["small"][1]
    q, s = quant.quant_rows(syn.f32_to_bf16_bits(vals).reshape(1, 128))
    assert s[0, 0] == np.float32(np.float32(32.0) / np.float32(448.0))
    assert list(q[0, :3]) == [0x7E, 0x46, 0x4E]
    assert list(e4m3.decode(q[0, :3])) == [448.0, 3.5, 7.0]


def test_per_tensor_outlier_claim_arithmetic():
    g = GOLDEN["per_tensor_outlier_example"]
    vals = np.full(128, g["normal"], np.float32)
    vals[0] = g["outlier"]
    q, s = quant.quant_rows(syn.f32_to_bf16_bits(vals).reshape(1, 128))
    # 0.5 / (120 / 448) = 1.867 -> 1.875, a normal E4M3 value (not subnormal)
    assert np.all(q[0, 1:] == 0x3F)
    assert e4m3.decode(np.uint8(0x3F)) == 1.875
    assert e4m3.decode(np.uint8(0x3F)) >= 2.0 ** -6


def test_drift_policies_invariants():
    seq = list(syn.drift_sequence(steps=100, M=128, K=1024, seed=0, spike_step=50))
    sig = [s for _, s, _ in seq]
    assert abs(sig[-1] / sig[0] - GOLDEN["drift_example"]["std_growth"]) < 1e-12
    res = policies.simulate(seq)
    cur, hist, fix = res["current"], res["history"], res["fixed"]
    assert all(r["saturated"] == 0 for r in cur)                 # online never clips
    for p in (hist, fix):                                        # all agree at step 0
        assert np.array_equal(p[0]["q"], cur[0]["q"]) and np.array_equal(p[0]["s"], cur[0]["s"])
    assert hist[50]["saturated"] > 0 and fix[50]["saturated"] > 0  # the spike clips
    assert np.array_equal(hist[1]["s"], fix[1]["s"])             # h_0 = amax_0
    summ = policies.summarize(res)
    assert summ["fixed"]["clip_rate"] > summ["history"]["clip_rate"] > 0
    # the history lags: its scales trail the online ones as the spread grows
    assert np.median(hist[99]["s"] / cur[99]["s"]) < 1.0


def test_history_update_no_fma():
    h = np.array([1.0, 3.0, 1e-30], np.float32)
    a = np.array([2.0, 0.0, 5.0], np.float32)
    out = policies.history_update(h, a)
    d = np.float32(0.9)
    want = (h * d).astype(np.float32) + (a * np.float32(np.float32(1) - d)).astype(np.float32)
    assert np.array_equal(out, want.astype(np.float32))
    assert np.float32(np.float32(1) - d) == np.float32(0.100000024)
