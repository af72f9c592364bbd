"""Scale policies over a drifting tile sequence (oracle; test infrastructure only).

Sources:

* "Online Quantization During Training": section 1 (a fixed scale taken
  from an early sample), section 2 (online: the scale follows the current
  tile), section 4 (delayed scaling / amax histories trade clipping for
  stability and lag behind fast shifts) and its worked example (a tile whose
  spread doubles over 100 steps with a rare 20-sigma outlier; compare fixed
  calibration, current-max and exponential amax history on clipping rate and
  mean error).
* "Introduction to LLM Quantization", section 5: delayed quantization derives
  the current scale from past maxima and can overflow when the range moves.
* "Online Quantization During Training", study lab: saturation through a
  curriculum change (``synthetic.curriculum_sequence``).

Policies, per 1x128 tile (readings where the pages are silent):

* ``current``: s_t from amax_t of the step itself (the online rule).
* ``history``: exponential amax history with decay 0.9.  h_0 = amax_0;
  after step t, h_t = fl32(fl32(0.9 * h_{t-1}) + fl32(fl32(1 - 0.9) * amax_t))
  (FP32, no fused multiply-add).  Step t >= 1 quantizes with
  s_t = max(fl32(h_{t-1} / 448), fl32(1e-12)), so step 0 equals ``current``.
* ``fixed``: the step-0 online scales, reused for every step.
* ``clip<r>`` (e.g. ``clip2``): percentile clipping of the current tile, the
  clip value being its r-th largest |x| (``oracle.granularity``).

Per step the oracle records the saturation count (elements whose rounded
scaled value lies beyond 448 before the clip, i.e. |fl32(x / s)| > 464), the
clipping rate
(count / elements) and the mean absolute reconstruction error
mean |x - q * s| (float64), also relative to mean |x|.
"""
from __future__ import annotations

import numpy as np

from . import e4m3, granularity, quant

DECAY = np.float32(0.9)


def history_update(h, amax, decay=DECAY):
    """h <- fl32(fl32(decay * h) + fl32(fl32(1 - decay) * amax)), elementwise FP32."""
    d = np.float32(decay)
    one_minus = np.float32(np.float32(1.0) - d)
    a = (np.asarray(h, np.float32) * d).astype(np.float32)
    b = (np.asarray(amax, np.float32) * one_minus).astype(np.float32)
    return (a + b).astype(np.float32)


def _step_stats(x_bits, q, s, sat):
    x = quant.bf16_to_f32(x_bits).astype(np.float64)
    M, K = x.shape
    deq = quant.dequant_rows(q, s)
    err = np.abs(x - deq)
    mean_abs = float(np.mean(np.abs(x)))
    return dict(saturated=int(sat), clip_rate=sat / x.size,
                mean_abs_err=float(np.mean(err)),
                rel_mean_abs_err=float(np.mean(err)) / mean_abs)


def simulate(sequence, policies=("current", "history", "fixed")):
    """Run the scale policies over ``sequence`` = iterable of (t, sigma, X_bits).

    Returns {policy: [per-step dict(saturated, clip_rate, mean_abs_err,
    rel_mean_abs_err, q, s)]}; q/s are the codes and scales used.
    """
    out = {p: [] for p in policies}
    hist = None
    fixed = None
    for t, _sigma, x_bits in sequence:
        q_cur, s_cur = quant.quant_rows(x_bits)
        _, amax, _ = quant.quant_rows_external(x_bits, s_cur)
        for p in policies:
            if p == "current":
                s = s_cur
            elif p == "history":
                s = s_cur if hist is None else quant.scale_from_amax(hist)
            elif p == "fixed":
                s = s_cur if fixed is None else fixed
            elif p.startswith("clip"):
                s = granularity.tile_scales(x_bits, 128, int(p[4:]))
            else:
                raise ValueError(p)
            q, _, sat = quant.quant_rows_external(x_bits, s)
            rec = _step_stats(x_bits, q, s, sat)
            rec["q"] = q
            rec["s"] = s
            out[p].append(rec)
        hist = amax.copy() if hist is None else history_update(hist, amax)
        if fixed is None:
            fixed = s_cur.copy()
    return out


def summarize(result):
    """Per-policy totals: overall clipping rate and mean relative error."""
    summary = {}
    for p, steps in result.items():
        sat = sum(r["saturated"] for r in steps)
        n = sum(r["q"].size for r in steps)
        summary[p] = dict(clip_rate=sat / n,
                          mean_rel_err=float(np.mean([r["rel_mean_abs_err"] for r in steps])),
                          saturated=sat)
    return summary


__all__ = ["simulate", "summarize", "history_update", "DECAY", "e4m3"]
