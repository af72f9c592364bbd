"""Caller-scale (delayed / history / fixed) quantization on the GPU, step by
step against the oracle's policy simulation: codes, per-tile amax and the
saturation count must match exactly at every one of the 100 steps.

The GPU chain is driven only by GPU outputs (its own amax_out feeds the
history-update kernel); the oracle chain only by the oracle.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import policies, quant

pytestmark = pytest.mark.gpu


def dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.int16) if t.dtype == torch.uint16 else t).cuda()


def test_history_update_kernel_matches_oracle(gpu_lib):
    rng = np.random.default_rng(0)
    h = (rng.random(5000) * 10).astype(np.float32)
    a = (rng.random(5000) * 10).astype(np.float32)
    a[:4] = [0.0, np.inf, 1e-40, 3e38]
    hd, ad = dev(h), dev(a)
    sd = torch.empty_like(hd)
    gpu_lib.amax_history_update(hd, ad, decay=0.9, scales_out=sd)
    torch.cuda.synchronize()
    want = policies.history_update(h, a)
    assert np.array_equal(hd.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert np.array_equal(sd.cpu().numpy().view(np.uint32),
                          quant.scale_from_amax(want).view(np.uint32))


def test_policies_100_steps_bit_exact(gpu_lib):
    M, K = 128, 7168
    seq = list(syn.drift_sequence(steps=100, M=M, K=K, seed=0, spike_step=50))
    ref = policies.simulate(seq)
    KB = K // 128
    hist = torch.zeros((KB, M), dtype=torch.float32, device="cuda")
    fixed = None
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    hist_scales = torch.empty_like(hist)
    for t, _sigma, xb in seq:
        x = dev(xb)
        q_cur, s_cur, amax = gpu_lib.quant_act_1x128(x, "row", return_amax=True)
        s_cur = s_cur[:, :M].contiguous()
        amax = amax[:, :M].contiguous()
        for p in ("current", "history", "fixed"):
            if p == "current" or t == 0:
                s = s_cur
            elif p == "history":
                s = hist_scales
            else:
                s = fixed
            sat.zero_()
            q, _, a2 = gpu_lib.quant_act_1x128(x, "row", scales_in=s, return_amax=True, sat_count=sat)
            torch.cuda.synchronize()
            r = ref[p][t]
            assert np.array_equal(q.cpu().numpy(), r["q"]), f"step {t} policy {p}: codes"
            assert np.array_equal(s.cpu().numpy().T.view(np.uint32), r["s"].view(np.uint32)), \
                f"step {t} policy {p}: scales"
            assert int(sat.item()) == r["saturated"], f"step {t} policy {p}: saturation count"
            assert torch.equal(a2, amax)
        if t == 0:
            gpu_lib.amax_history_update(hist, amax, decay=0.9, init=True, scales_out=hist_scales)
            fixed = s_cur.clone()
        else:
            gpu_lib.amax_history_update(hist, amax, decay=0.9, scales_out=hist_scales)
    summ = policies.summarize(ref)
    assert summ["current"]["saturated"] == 0 and summ["fixed"]["saturated"] > 0


def test_curriculum_policies_bit_exact(gpu_lib):
    """Saturation through a curriculum change (sigma 1 -> 4 at step 40 -> 1 at
    step 70) for the online, history, fixed and 2nd-largest-clip policies,
    every step bit-exact with the oracle; the per-step counts are printed."""
    M, K = 128, 7168
    seq = list(syn.curriculum_sequence(steps=100, M=M, K=K, seed=0))
    pols = ("current", "history", "fixed", "clip2")
    ref = policies.simulate(seq, pols)
    KB = K // 128
    hist = torch.zeros((KB, M), dtype=torch.float32, device="cuda")
    hist_scales = torch.empty_like(hist)
    fixed = None
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    counts = {p: [] for p in pols}
    for t, _sigma, xb in seq:
        x = dev(xb)
        _, s_cur, amax = gpu_lib.quant_act_1x128(x, "row", return_amax=True)
        s_cur = s_cur[:, :M].contiguous()
        amax = amax[:, :M].contiguous()
        for p in pols:
            sat.zero_()
            if p == "clip2":
                q, s = gpu_lib.quant_act_tiles(x, 128, 2, sat_count=sat)
                s = s[:, :M]
            else:
                s = s_cur if (p == "current" or t == 0) else (hist_scales if p == "history" else fixed)
                q, _, _ = gpu_lib.quant_act_1x128(x, "row", scales_in=s, sat_count=sat)
            torch.cuda.synchronize()
            r = ref[p][t]
            assert np.array_equal(q.cpu().numpy(), r["q"]), f"step {t} policy {p}: codes"
            assert np.array_equal(s.cpu().numpy().T.view(np.uint32), r["s"].view(np.uint32)), \
                f"step {t} policy {p}: scales"
            assert int(sat.item()) == r["saturated"], f"step {t} policy {p}: saturation count"
            counts[p].append(int(sat.item()))
        if t == 0:
            gpu_lib.amax_history_update(hist, amax, decay=0.9, init=True, scales_out=hist_scales)
            fixed = s_cur.clone()
        else:
            gpu_lib.amax_history_update(hist, amax, decay=0.9, scales_out=hist_scales)
    print("\nstep  " + "  ".join(f"{p:>8s}" for p in pols))
    for t in list(range(0, 100, 5)) + [41, 42, 43, 71]:
        print(f"{t:4d}  " + "  ".join(f"{counts[p][t]:8d}" for p in pols))
    assert sum(counts["current"]) == 0
    assert counts["history"][40] > 20 * np.mean(counts["history"][10:40])
