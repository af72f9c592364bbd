"""Pins for the policy simulation through a curriculum change (CPU only).

The sequence keeps sigma = 1, jumps to 4 at step 40 and back to 1 at step
70.  Pinned by what the definitions force: online scales never saturate;
the fixed step-0 scales saturate many times more during the 4x stretch than
before or after it; the amax history saturates most at the jump, falls as
it catches up, and not at all right after the drop (its scales are then too
large); clipping at the 2nd largest value saturates at most one value per
tile; clip1 is the online rule.
"""
import numpy as np

from oracle import granularity, policies, quant
import synthetic as syn


def _run(steps=100, M=32, K=1024, pol=("current", "history", "fixed", "clip1", "clip2")):
    seq = list(syn.curriculum_sequence(steps=steps, M=M, K=K, seed=0))
    return seq, policies.simulate(seq, pol)


def test_curriculum_sigmas():
    sig = [s for _, s, _ in syn.curriculum_sequence(steps=100, M=4, K=128)]
    assert sig[:40] == [1.0] * 40 and sig[40:70] == [4.0] * 30 and sig[70:] == [1.0] * 30


def test_curriculum_saturation_pattern():
    seq, r = _run()
    sat = {p: np.array([s["saturated"] for s in r[p]]) for p in r}
    ntiles = 32 * 1024 // 128
    assert not sat["current"].any()
    assert np.array_equal(sat["clip1"], sat["current"])
    # a fresh draw per step: step-0 or history scales are exceeded by some
    # tiles even at a steady sigma; the 4x stretch multiplies that many-fold
    calm = sat["fixed"][1:40].mean()
    assert sat["fixed"][40:70].min() > 20 * calm
    assert sat["fixed"][70:].mean() < 2 * calm
    steady = sat["history"][10:40].mean()
    assert sat["history"][40] > 20 * steady
    assert sat["history"][69] < sat["history"][40] / 5      # the history catches up
    assert not sat["history"][70:75].any()                  # too-large scales after the drop
    # clipping at the 2nd largest |x|: only a tile's largest value can saturate
    assert np.all(sat["clip2"] > 0) and np.all(sat["clip2"] <= ntiles)


def test_clip1_codes_equal_online():
    seq, r = _run(steps=3, M=16, K=512, pol=("current", "clip1"))
    for a, b in zip(r["current"], r["clip1"]):
        assert np.array_equal(a["q"], b["q"]) and np.array_equal(a["s"], b["s"])
    s1 = granularity.tile_scales(seq[2][2], 128, 1)
    assert np.array_equal(r["clip1"][2]["s"], s1)
