"""Pins for the oracle's FP8 token payloads (CPU only).

Pinned by: the message size in closed form (half of BF16 plus one scale per
128 values), a message built by hand byte by byte (code values, scale bits,
byte order, scale position), lossless tiles that must come back bit for bit,
gathering against packing the permuted input, the NaN message of an invalid
source row, and BF16 restoration against exact rational round-to-nearest-even
over every code, including products that FP32 would first round onto a BF16
tie (a double-rounding trap).
"""
from fractions import Fraction

import numpy as np

from oracle import e4m3, payload, quant
import synthetic as syn


def test_message_bytes_closed_form():
    # H codes + H/128 four-byte scales; 7168 -> 7168 + 224
    assert payload.message_bytes(7168) == 7392
    assert payload.message_bytes(128) == 132
    # against BF16 (2 bytes per value): (1 + 4/128) / 2 = 33/64 for any H
    for H in (128, 1024, 7168):
        assert Fraction(payload.message_bytes(H), 2 * H) == Fraction(33, 64)


def test_hand_built_message():
    # one token, H = 128: amax 56 -> scale 56/448 = 1/8 (FP32 0x3E000000)
    # 56 -> 448 (0x7E), 0.125 -> 1.0 (0x38), -0.125 -> -1.0 (0xB8), 0 -> 0x00,
    # 2**-10 -> 2**-7, below the smallest normal 2**-6: subnormal 4 * 2**-9 = 0x04
    row = np.zeros(128, np.float32)
    row[0], row[1], row[2], row[5] = 56.0, 0.125, -0.125, 2.0 ** -10
    msg = payload.pack_tokens(syn.f32_to_bf16_bits(row[None, :]))
    assert msg.shape == (1, 132)
    want = np.zeros(132, np.uint8)
    want[0], want[1], want[2], want[5] = 0x7E, 0x38, 0xB8, 0x04
    want[128:132] = [0x00, 0x00, 0x00, 0x3E]                     # little-endian 0x3E000000
    assert np.array_equal(msg[0], want)


def test_stride_padding_is_zero():
    x = syn.activation_with_outliers(8, 256, seed=5)
    m = payload.pack_tokens(x, stride=272)
    assert m.shape == (8, 272) and not m[:, 264:].any()
    assert np.array_equal(m[:, :264], payload.pack_tokens(x))


def test_lossless_round_trip_and_known_scales():
    bits, k = syn.lossless_tiles(48, 1024, seed=11, tile=(1, 128))
    msgs = payload.pack_tokens(bits)
    q, s = payload.unpack_tokens(msgs, 1024)
    assert np.array_equal(s, np.exp2(k).astype(np.float32))       # s = 2**k per tile
    assert np.array_equal(payload.dequant_tokens(msgs, 1024), bits)  # every value comes back


def test_unpacked_codes_are_the_row_quantization():
    x = syn.activation_with_outliers(40, 896, seed=7)
    q, s = payload.unpack_tokens(payload.pack_tokens(x), 896)
    q0, s0 = quant.quant_rows(x)
    assert np.array_equal(q, q0) and np.array_equal(s.view(np.uint32), s0.view(np.uint32))


def test_gather_equals_packing_the_permuted_rows():
    x = syn.activation_with_outliers(64, 512, seed=8)
    src = syn.dispatch_rows(64, 8, 3, seed=2)
    assert len(src) == 192 and np.array_equal(np.bincount(src), np.full(64, 3))
    assert np.array_equal(payload.pack_tokens(x, src), payload.pack_tokens(x[src]))


def test_invalid_source_row_gives_nan_message():
    x = syn.gaussian((4, 256), seed=1)
    m = payload.pack_tokens(x, np.array([1, -1, 4, 3]))
    for t in (1, 2):
        assert np.all(m[t, :256] == 0x7F)
        assert np.all(m[t, 256:].view("<u4") == 0x7FC00000)
    assert np.array_equal(m[[0, 3]], payload.pack_tokens(x[[1, 3]]))


def _rne_bf16_bits(code: int, scale: np.float32) -> int:
    """Exact rational q * s rounded to BF16 (nearest, ties to even)."""
    neg = bool(code & 0x80)
    mag = Fraction(float(e4m3.decode(np.uint8(code & 0x7F)))) * Fraction(float(scale))
    if mag == 0:
        return 0x8000 if neg else 0
    e = mag.numerator.bit_length() - mag.denominator.bit_length()
    if Fraction(2) ** e > mag:
        e -= 1
    spacing = Fraction(2) ** (max(e, -126) - 7)
    n = mag / spacing
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    v = float(lo * spacing)
    bits = int(np.array(v, np.float32).view(np.uint32)) >> 16
    return bits | (0x8000 if neg else 0)


def _double_rounding_traps():
    """(code, scale) whose exact product is not a BF16 midpoint but rounds to
    one in FP32."""
    out = []
    for qv in (1.125, 1.375, 0.875, 5.0):
        code = int(e4m3.encode(np.float32(qv)))
        for j in (1, 3, 5, 7, 21, 40, 63):
            mid = 1.0 + (2 * j - 1) * 2.0 ** -8
            s = np.float32(mid / qv)
            for _ in range(12):
                s = np.nextafter(s, np.float32(np.inf))
                p = qv * float(s)
                if p != mid and float(np.float32(p)) == mid:
                    out.append((code, np.float32(s)))
            s = np.float32(mid / qv)
            for _ in range(12):
                s = np.nextafter(s, np.float32(-np.inf))
                p = qv * float(s)
                if p != mid and float(np.float32(p)) == mid:
                    out.append((code, np.float32(s)))
    return out


def test_dequant_is_exact_rne_over_every_code():
    scales = [np.float32(v) for v in (1.0, 0.125, 2.0 ** -20, 3.0e-5, 0.7071067690849304, 1.3e30)]
    traps = _double_rounding_traps()
    assert len(traps) >= 8
    pairs = [(c, s) for s in scales for c in range(256) if (c & 0x7F) != 0x7F] + traps
    H = 128
    msgs = np.zeros((len(pairs), H + 4), np.uint8)
    want = np.zeros((len(pairs), H), np.uint16)
    for i, (c, s) in enumerate(pairs):
        msgs[i, :H] = c
        msgs[i, H:] = np.array([s], "<f4").view(np.uint8)
        want[i, :] = _rne_bf16_bits(c, s)
    got = payload.dequant_tokens(msgs, H)
    assert np.array_equal(got, want)
    # the traps really differ from FP32-then-BF16 rounding somewhere
    naive = [(int(np.array(np.float32(float(e4m3.decode(np.uint8(c))) * float(s)), np.float32).view(np.uint32)))
             for c, s in traps]
    tie_even = [((b + 0x7FFF + ((b >> 16) & 1)) >> 16) & 0xFFFF for b in naive]
    assert any(t != int(want[len(pairs) - len(traps) + i, 0]) for i, t in enumerate(tie_even))


def test_nan_codes_restore_to_nan():
    msgs = np.zeros((1, 132), np.uint8)
    msgs[0, :2] = [0x7F, 0xFF]
    msgs[0, 128:] = np.array([1.0], "<f4").view(np.uint8)
    out = payload.dequant_tokens(msgs, 128)
    assert out[0, 0] == 0x7FC0 and out[0, 1] == 0x7FC0 and out[0, 2] == 0
