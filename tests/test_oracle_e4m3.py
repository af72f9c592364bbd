"""Pins for the oracle's E4M3 codec (CPU only).

The codec is pinned to what the pages fix (1-4-3 bit split, largest value
448, clip to +-448) and to independent references: exact rational
nearest-value search, the closed-form grid, and PyTorch's CPU float8_e4m3fn
cast (after an explicit clamp, because that cast does not saturate).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def test_page_max_and_bit_split():
    g = GOLDEN["e4m3_bits"]
    assert g["sign"] + g["exponent"] + g["mantissa"] == 8
    assert e4m3.decode(np.uint8(0x7E)) == GOLDEN["e4m3_max"]["value"]
    assert e4m3.decode(np.uint8(0xFE)) == -GOLDEN["e4m3_max"]["value"]
    assert np.nanmax(e4m3.DECODE_TABLE) == 448.0
    assert e4m3.encode(np.float32(448.0)) == 0x7E


def test_table_structure():
    vals = e4m3.DECODE_TABLE
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    finite = vals[np.isfinite(vals)]
    assert finite.size == 254
    assert np.unique(finite).size == 253          # +0 and -0 coincide
    # closed forms: smallest subnormal, smallest normal, largest subnormal, 1.0
    assert vals[0x01] == 2.0 ** -9
    assert vals[0x07] == 7 * 2.0 ** -9
    assert vals[0x08] == 2.0 ** -6
    assert vals[0x38] == 1.0
    # every finite value is an integer multiple of 2**-9 (used by the GEMM exactness proof)
    assert np.all(np.mod(finite * 2 ** 9, 1.0) == 0)
    # sign symmetry
    assert np.array_equal(vals[0x80:0xFF], -vals[0x00:0x7F])


def test_decode_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = e4m3.encode(e4m3.decode(codes).astype(np.float32))
    assert np.array_equal(back, codes)             # keeps the sign of zero
    assert e4m3.encode(np.float32(np.nan)) == 0x7F


def _nearest_exact(y: float) -> int:
    """Nearest E4M3 code by exact rational search; ties to even code."""
    if np.isnan(y):
        return 0x7F
    a = min(Fraction(abs(float(y))), Fraction(448))
    grid = [Fraction(float(v)) for v in e4m3.GRID]
    dists = [abs(a - g) for g in grid]
    best = min(dists)
    cands = [i for i, d in enumerate(dists) if d == best]
    code = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return code | (0x80 if np.signbit(y) else 0)


def test_midpoints_ties_and_neighbours():
    mids = e4m3.MIDPOINTS.astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), e4m3.MIDPOINTS)   # midpoints are fp32-exact
    got = e4m3.encode(mids)
    want = np.array([_nearest_exact(m) for m in mids])
    assert np.array_equal(got, want)
    assert np.all(got % 2 == 0)                    # ties go to the even code
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    assert np.array_equal(e4m3.encode(up), np.arange(1, 127))
    assert np.array_equal(e4m3.encode(dn), np.arange(0, 126))
    # pinned ties: 2**-10 -> 0x00, 3 * 2**-11 -> 0x01, 464 -> 0x7E
    assert e4m3.encode(np.float32(2.0 ** -10)) == 0x00
    assert e4m3.encode(np.float32(3 * 2.0 ** -11)) == 0x01
    assert e4m3.encode(np.float32(464.0)) == 0x7E


def test_saturation_and_specials():
    ys = np.array([448.5, 463.99, 464, 465, 1e30, np.inf, 3.4e38], dtype=np.float32)
    assert np.all(e4m3.encode(ys) == 0x7E)
    assert np.all(e4m3.encode(-ys) == 0xFE)
    assert e4m3.encode(np.float32(-0.0)) == 0x80
    assert e4m3.encode(np.float32(-1e-30)) == 0x80
    assert e4m3.encode(np.float32(1e-45)) == 0x00
    assert e4m3.encode(f32(0xFFC00000)) == 0x7F     # any NaN -> canonical NaN code


def test_rational_search_on_random_fp32():
    rng = np.random.default_rng(1)
    e = rng.integers(110, 137, size=3000)
    bits = (e << 23) | rng.integers(0, 1 << 23, size=3000)
    bits |= rng.integers(0, 2, size=3000) << 31
    ys = f32(bits)
    got = e4m3.encode(ys)
    want = np.array([_nearest_exact(y) for y in ys])
    assert np.array_equal(got, want)


def _torch_ref(ys):
    t = torch.from_numpy(np.asarray(ys, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_agrees_with_torch_cast_after_clamp():
    # every BF16 pattern widened to fp32, plus dense random fp32 bit patterns
    bf = (np.arange(1 << 16, dtype=np.uint32) << 16)
    rng = np.random.default_rng(2)
    rnd = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # and the fp32 neighbourhood of every midpoint
    mids = e4m3.MIDPOINTS.astype(np.float32).view(np.uint32)
    near = (mids[:, None].astype(np.int64) + np.arange(-3, 4)[None, :]).ravel().astype(np.uint32)
    near = np.concatenate([near, near | np.uint32(0x80000000)])
    ys = f32(np.concatenate([bf, rnd, near]))
    ys = ys[~np.isnan(ys)]
    assert np.array_equal(e4m3.encode(ys), _torch_ref(ys))


def test_monotone_over_structured_fp32_sweep():
    # all fp32 patterns whose low 12 mantissa bits take 4 boundary values
    hi = np.arange(0, 1 << 19, dtype=np.uint32) << 12
    lows = np.array([0, 1, 0x7FF, 0x800, 0xFFF], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    ys = f32(bits)
    ys = np.sort(ys[np.isfinite(ys)])
    v = e4m3.decode(e4m3.encode(ys))
    assert np.all(np.diff(v) >= 0)


@pytest.mark.parametrize("value,code", [(1.0, 0x38), (1.875, 0x3F), (3.5, 0x46), (7.0, 0x4E),
                                        (0.015625, 0x08), (240.0, 0x77), (256.0, 0x78)])
def test_closed_form_codes(value, code):
    assert e4m3.encode(np.float32(value)) == code
    assert e4m3.decode(np.uint8(code)) == value
