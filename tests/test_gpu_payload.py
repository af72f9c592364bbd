"""GPU parity of the FP8 token payloads against the oracle (bit-exact).

Packing is checked byte for byte against ``oracle.payload`` (ragged token
counts, adversarial tiles, gathering with repeated and invalid source rows,
padded strides); unpacking must give exactly the row quantizer's operand
layout; BF16 restoration is checked over every code with scales that reach
the kernel's integer path (tiny and subnormal FP32 scales) and with products
that FP32 would round onto a BF16 midpoint.  The full-size case packs the
dispatch of 4096 tokens x 7168 channels to 8 experts (top-8 of 8 is every
expert; top-2 here) and compares a seeded sample of messages.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import e4m3, payload
from test_gpu_quant import adversarial_rows

pytestmark = pytest.mark.gpu


def dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.cuda()


def host(t):
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy()


def check_pack(fp8, x, src=None, stride=None, label=""):
    H = x.shape[1]
    mb = payload.message_bytes(H)
    src_t = None if src is None else dev(np.asarray(src, np.int32))
    msg = fp8.pack_tokens(dev(x), src_t, stride=stride)
    torch.cuda.synchronize()
    got = host(msg)[:, :mb]
    want = payload.pack_tokens(x, src)[:, :mb]
    bad = np.nonzero(np.any(got != want, axis=1))[0]
    assert bad.size == 0, f"{label}: {bad.size} messages differ, first {bad[:5]}"
    return msg


@pytest.mark.parametrize("case", ["ragged", "adversarial", "lossless", "gather", "invalid", "stride"])
def test_pack_small(gpu_lib, case):
    if case == "ragged":
        check_pack(gpu_lib, syn.activation_with_outliers(37, 2304, seed=21), label=case)
    elif case == "adversarial":
        check_pack(gpu_lib, adversarial_rows(), label=case)
    elif case == "lossless":
        x, _ = syn.lossless_tiles(19, 640, seed=22, tile=(1, 128))
        check_pack(gpu_lib, x, label=case)
    elif case == "gather":
        x = syn.activation_with_outliers(96, 1024, seed=23)
        check_pack(gpu_lib, x, syn.dispatch_rows(96, 8, 3, seed=4), label=case)
    elif case == "invalid":
        x = syn.gaussian((10, 384), seed=24)
        check_pack(gpu_lib, x, [3, -1, 10, 9, 0, 2**31 - 1, -(2**31), 5], label=case)
    else:
        x = syn.activation_with_outliers(21, 896, seed=25)
        check_pack(gpu_lib, x, stride=1024, label=case)


def test_unpack_is_the_row_operand(gpu_lib):
    x = syn.activation_with_outliers(150, 1792, seed=26)
    msg = gpu_lib.pack_tokens(dev(x))
    q, s = gpu_lib.unpack_tokens(msg, 1792)
    q0, s0, _ = gpu_lib.quant_act_1x128(dev(x), "row")
    torch.cuda.synchronize()
    assert torch.equal(q, q0)
    assert np.array_equal(host(s)[:, :150].view(np.uint32), host(s0)[:, :150].view(np.uint32))
    # and against the oracle's unpacking of the oracle's messages
    qo, so = payload.unpack_tokens(payload.pack_tokens(x), 1792)
    assert np.array_equal(host(q), qo)
    assert np.array_equal(host(s)[:, :150].T.view(np.uint32), so.view(np.uint32))


def _dequant_fixture():
    """Messages (H = 128) covering every code under many scales."""
    scales = [1.0, 0.125, 3.0e-5, 0.7071067690849304, 1.3e30, 3.0e38,
              2.0 ** -117, 2.0 ** -118, 2.0 ** -120, 1.1754942e-38, 2.0 ** -130, 2.0 ** -149,
              3.3e-42, 0.0, -0.0, -2.5, np.inf, -np.inf, np.nan]
    rows = []
    for s in scales:
        for c0 in (0, 128):
            m = np.zeros(132, np.uint8)
            m[:128] = np.arange(c0, c0 + 128, dtype=np.uint8)
            m[128:] = np.array([s], "<f4").view(np.uint8)
            rows.append(m)
    # FP32 double-rounding traps: exact product just off a BF16 midpoint
    for qv in (1.125, 1.375, 0.875, 5.0, 0.0703125):
        code = int(e4m3.encode(np.float32(qv)))
        for j in (1, 3, 5, 7, 21, 40, 63):
            mid = 1.0 + (2 * j - 1) * 2.0 ** -8
            for direction in (np.inf, -np.inf):
                s = np.float32(mid / qv)
                for _ in range(12):
                    s = np.nextafter(s, np.float32(direction))
                    p = qv * float(s)
                    if p != mid and float(np.float32(p)) == mid:
                        m = np.full(132, code, np.uint8)
                        m[1::2] = code | 0x80
                        m[128:] = np.array([s], "<f4").view(np.uint8)
                        rows.append(m)
    out = np.zeros((len(rows), 144), np.uint8)          # stride: a multiple of 16
    out[:, :132] = np.stack(rows)
    return out


def test_dequant_every_code_and_scale(gpu_lib):
    msgs = _dequant_fixture()
    assert msgs.shape[0] > 40
    y = gpu_lib.dequant_tokens(dev(msgs), 128)
    torch.cuda.synchronize()
    got = host(y).view(np.uint16)
    want = payload.dequant_tokens(msgs, 128)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} values differ, first (msg, col) {bad[:4].tolist()}"


def test_round_trip_restores_lossless_tiles(gpu_lib):
    x, _ = syn.lossless_tiles(64, 2048, seed=27, tile=(1, 128))
    y = gpu_lib.dequant_tokens(gpu_lib.pack_tokens(dev(x)), 2048)
    torch.cuda.synchronize()
    assert np.array_equal(host(y).view(np.uint16), x)


def test_dispatch_full_size_sampled(gpu_lib):
    T, H = 4096, 7168
    x = syn.activation_with_outliers(T, H, seed=1)
    src = syn.dispatch_rows(T, 8, 2, seed=5)
    msg = gpu_lib.pack_tokens(dev(x), dev(src))
    y = gpu_lib.dequant_tokens(msg, H)
    q, s = gpu_lib.unpack_tokens(msg, H)
    torch.cuda.synchronize()
    assert msg.shape == (T * 2, 7392)
    pick = np.sort(np.random.default_rng(9).choice(T * 2, 192, replace=False))
    want = payload.pack_tokens(x, src[pick])
    got = host(msg[torch.from_numpy(pick).cuda()])
    assert np.array_equal(got, want)
    assert np.array_equal(host(y[torch.from_numpy(pick).cuda()]).view(np.uint16),
                          payload.dequant_tokens(want, H))
    qo, so = payload.unpack_tokens(want, H)
    assert np.array_equal(host(q[torch.from_numpy(pick).cuda()]), qo)
    assert np.array_equal(host(s)[:, pick].T.view(np.uint32), so.view(np.uint32))
