"""Thin PyTorch-facing binding of libfp8bs.so (argument marshalling only).

Tensors are used for device memory and the current HIP stream; every step of
the computation runs in the library's kernels.  Names follow the C ABI in
include/fp8bs.h.  Scale arrays are MN-major: [K/128][ld] with
ld = round_up(rows, 4) for 1x128 row tiles.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

FP8_DTYPE = torch.uint8


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t):
    return None if t is None else ctypes_ptr(t)


def ctypes_ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _check_2d(name, t, dtypes):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name}: expected a 2-D row-major tensor, got shape {tuple(t.shape)} "
                         f"strides {t.stride()}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def quant_act_1x128(x: torch.Tensor, direction: str = "row", *, scales_in=None,
                    return_amax: bool = False, sat_count=None, out=None, scales_out=None, stream=None):
    """Online FP8 quantization of activations.

    direction "row": 1x128 tiles along each row; returns
        q [rows][cols] uint8, scales [cols/128][round_up(rows, 4)] float32.
    direction "col": 128x1 tiles along each column, transposed output; returns
        q [cols][rows] uint8, scales [rows/128][round_up(cols, 4)] float32.
    direction "col_tiled": as "col" with q holding the operand-tiled bytes of
        the transposed codes (for the "wgrad_tiled" GEMM layout).
    scales_in (row only): caller scales in the scale layout; then the returned
    scales are None.  return_amax adds the per-tile max |x| (same layout).
    sat_count: optional int32/uint32 device tensor of one element, incremented.
    out / scales_out: optional caller buffers for q (the shape above, uint8)
    and the scales (at least the shape above, float32, row-major; its row
    stride is passed as ld_s), so that repeated calls allocate nothing.
    Returns (q, scales, amax_or_None).
    """
    lib = _lib.load_library()
    _check_2d("x", x, _BF16)
    rows, cols = x.shape
    dev = x.device
    if direction == "row":
        q_shape = (rows, cols)
        s_shape = (cols // 128, round_up(rows, 4))
        tile_dir = _lib.TILE_ROW
    elif direction in ("col", "col_tiled"):
        q_shape = (cols, rows)
        s_shape = (rows // 128, round_up(cols, 4))
        tile_dir = _lib.TILE_COL if direction == "col" else _lib.TILE_COL_TILED
    else:
        raise ValueError(direction)
    if out is None:
        q = torch.empty(q_shape, dtype=torch.uint8, device=dev)
    else:
        _check_2d("out", out, (torch.uint8, torch.float8_e4m3fn))
        if tuple(out.shape) != q_shape or not out.is_contiguous():
            raise ValueError(f"out: expected a contiguous {q_shape} tensor, got {tuple(out.shape)}")
        q = out
    if scales_in is not None:
        _check_2d("scales_in", scales_in, (torch.float32,))
        scales = None
        ld_s = scales_in.stride(0)
    elif scales_out is not None:
        _check_2d("scales_out", scales_out, (torch.float32,))
        if scales_out.shape[0] < s_shape[0] or scales_out.shape[1] < s_shape[1]:
            raise ValueError(f"scales_out: expected at least {s_shape}, got {tuple(scales_out.shape)}")
        scales = scales_out
        ld_s = scales_out.stride(0)
    else:
        scales = torch.empty(s_shape, dtype=torch.float32, device=dev)
        ld_s = s_shape[1]
    amax = torch.empty(s_shape if scales_in is None else tuple(scales_in.shape),
                       dtype=torch.float32, device=dev) if return_amax else None
    st = lib.fp8_quant_act_1x128(
        _ptr(x), rows, cols, x.stride(0), tile_dir, _ptr(q), q.stride(0),
        _ptr(scales), ld_s, _ptr(scales_in), _ptr(amax), _ptr(sat_count), _stream(stream))
    _lib.check("fp8_quant_act_1x128", st)
    return q, scales, amax


def quant_act_dual(x: torch.Tensor, *, tiled: bool = False, stream=None):
    """Both orientations of x [rows][cols] BF16 from one read.

    Returns (q_row [rows][cols], s_row [cols/128][round_up(rows, 4)],
             q_col [cols][rows], s_col [rows/128][round_up(cols, 4)]) - the outputs of
    quant_act_1x128(x, "row") and quant_act_1x128(x, "col") ("col_tiled" if tiled).
    """
    lib = _lib.load_library()
    _check_2d("x", x, _BF16)
    rows, cols = x.shape
    q_row = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s_row = torch.empty((cols // 128, round_up(rows, 4)), dtype=torch.float32, device=x.device)
    q_col = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    s_col = torch.empty((rows // 128, round_up(cols, 4)), dtype=torch.float32, device=x.device)
    if tiled:
        st = lib.fp8_quant_act_dual_tiled(_ptr(x), rows, cols, x.stride(0), _ptr(q_row), q_row.stride(0),
                                          _ptr(s_row), s_row.stride(0), _ptr(q_col), _ptr(s_col),
                                          s_col.stride(0), _stream(stream))
        _lib.check("fp8_quant_act_dual_tiled", st)
        return q_row, s_row, q_col, s_col
    st = lib.fp8_quant_act_dual(_ptr(x), rows, cols, x.stride(0), _ptr(q_row), q_row.stride(0),
                                _ptr(s_row), s_row.stride(0), _ptr(q_col), q_col.stride(0),
                                _ptr(s_col), s_col.stride(0), _stream(stream))
    _lib.check("fp8_quant_act_dual", st)
    return q_row, s_row, q_col, s_col


def quant_weight_128x128(w: torch.Tensor, *, transposed: bool = False, tiled: bool = False,
                         stream=None):
    """128x128 block quantization of weights [N][K].

    Returns (q [N][K] uint8, scales [N/128][K/128] float32, q_t [K][N] or None).
    tiled: q (and q_t) hold the operand-tiled bytes of the same codes, for
    the "fprop_tiled" / "dgrad_t_tiled" GEMM layouts (same shapes).
    """
    lib = _lib.load_library()
    _check_2d("w", w, _BF16)
    rows, cols = w.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=w.device)
    q_t = torch.empty((cols, rows), dtype=torch.uint8, device=w.device) if transposed else None
    scales = torch.empty((rows // 128, cols // 128), dtype=torch.float32, device=w.device)
    if tiled:
        st = lib.fp8_quant_weight_128x128_tiled(_ptr(w), rows, cols, w.stride(0), _ptr(q), _ptr(q_t),
                                                _ptr(scales), scales.stride(0), _stream(stream))
        _lib.check("fp8_quant_weight_128x128_tiled", st)
        return q, scales, q_t
    st = lib.fp8_quant_weight_128x128(
        _ptr(w), rows, cols, w.stride(0), _ptr(q), q.stride(0), _ptr(q_t),
        q_t.stride(0) if q_t is not None else 0, _ptr(scales), scales.stride(0), _stream(stream))
    _lib.check("fp8_quant_weight_128x128", st)
    return q, scales, q_t


def block_gemm_noalloc(layout: str, A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor, sB: torch.Tensor,
                       *, out, stream=None):
    """block_gemm through fp8_block_gemm_noalloc: the library allocates
    nothing (its split workspace is a static device array shared by every call
    on the GPU; calls that overlap in time on one GPU race).  `out` is the
    caller's C [M][N] (bfloat16 or float32)."""
    return block_gemm(layout, A, sA, B, sB, out=out, stream=stream, _entry="fp8_block_gemm_noalloc")


def block_gemm(layout: str, A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor, sB: torch.Tensor,
               *, out_dtype=torch.bfloat16, out=None, stream=None, _entry="fp8_block_gemm"):
    """Block-scaled FP8 GEMM.

    fprop: A [M][K], sA [K/128][>=M], B [N][K], sB [N/128][>=K/128]
    dgrad: A [M][K], sA [K/128][>=M], B [K][N] (forward W_q), sB [K/128][>=N/128]
    dgrad_t: A [M][K], sA [K/128][>=M], B [N][K] (W_q^T, the q_t of the weight
             quantizer), sB [K/128][>=N/128] (the forward block-scale table)
    wgrad: A [M][K], sA [K/128][>=M], B [N][K], sB [K/128][>=N]
    fprop_tiled / dgrad_t_tiled / wgrad_tiled: as fprop / dgrad_t / wgrad with
             B holding the operand-tiled bytes (quant_weight_128x128(...,
             tiled=True); for wgrad quant_act_1x128(x, "col_tiled") or
             quant_act_dual(x, tiled=True))
    Returns C [M][N] in out_dtype (bfloat16 or float32).
    """
    lib = _lib.load_library()
    for n, t in (("A", A), ("B", B)):
        _check_2d(n, t, (torch.uint8, torch.float8_e4m3fn))
    _check_2d("sA", sA, (torch.float32,))
    _check_2d("sB", sB, (torch.float32,))
    M, K = A.shape
    N = B.shape[1] if layout == "dgrad" else B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    code = _lib.OUT_FP32 if out.dtype == torch.float32 else _lib.OUT_BF16
    st = getattr(lib, _entry)(
        _lib.LAYOUT[layout], M, N, K, _ptr(A), A.stride(0), _ptr(sA), sA.stride(0),
        _ptr(B), B.stride(0), _ptr(sB), sB.stride(0), _ptr(out), code, out.stride(0),
        _stream(stream))
    _lib.check(_entry, st)
    return out


def block_gemm_fused_quant(x: torch.Tensor, W: torch.Tensor, sW: torch.Tensor, *, out_dtype=torch.bfloat16,
                           with_codes: bool = False, out=None, stream=None):
    """Fprop with the 1x128 quantization of X fused into the GEMM.

    x: bfloat16 [M][K]; W: codes [N][K] (row-major); sW [N/128][>=K/128].
    Returns C [M][N] (out_dtype), equal bit for bit to
    block_gemm("fprop", *quant_act_1x128(x, "row")[:2], W, sW); with
    with_codes=True returns (C, codes [M][K], scales [K/128][M_pad]) as the
    kernel formed them.
    """
    lib = _lib.load_library()
    _check_2d("x", x, _BF16)
    _check_2d("W", W, (torch.uint8, torch.float8_e4m3fn))
    _check_2d("sW", sW, (torch.float32,))
    M, K = x.shape
    N = W.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    code = _lib.OUT_FP32 if out.dtype == torch.float32 else _lib.OUT_BF16
    q = s = None
    if with_codes:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        s = torch.empty((K // 128, round_up(M, 4)), dtype=torch.float32, device=x.device)
    st = lib.fp8_block_gemm_fused_quant(
        M, N, K, _ptr(x), x.stride(0), _ptr(W), W.stride(0), _ptr(sW), sW.stride(0), _ptr(out), code,
        out.stride(0), _ptr(q) if q is not None else None, q.stride(0) if q is not None else 0,
        _ptr(s) if s is not None else None, s.stride(0) if s is not None else 0, _stream(stream))
    _lib.check("fp8_block_gemm_fused_quant", st)
    return (out, q, s) if with_codes else out


def block_gemm_grouped(offsets: torch.Tensor, A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor,
                       sB: torch.Tensor, *, tiled: bool = False, out_dtype=torch.bfloat16, out=None,
                       stream=None):
    """Grouped per-expert Fprop in one launch.

    offsets: int32 device [G+1]; A [total_M][K]; sA [K/128][>=total_M];
    B [G][N][K] (operand-tiled bytes per expert if tiled); sB [G][N/128][K/128].
    Returns C [total_M][N].
    """
    lib = _lib.load_library()
    _check_2d("A", A, (torch.uint8, torch.float8_e4m3fn))
    _check_2d("sA", sA, (torch.float32,))
    if B.dim() != 3 or not B.is_contiguous() or sB.dim() != 3 or not sB.is_contiguous():
        raise ValueError("B must be contiguous [G][N][K] and sB contiguous [G][N/128][K/128]")
    if offsets.dtype != torch.int32 or not offsets.is_cuda:
        raise TypeError("offsets must be an int32 device tensor")
    G, N, K = B.shape
    total_M = A.shape[0]
    if out is None:
        out = torch.empty((total_M, N), dtype=out_dtype, device=A.device)
    code = _lib.OUT_FP32 if out.dtype == torch.float32 else _lib.OUT_BF16
    if tiled:
        st = lib.fp8_block_gemm_grouped_tiled(
            G, _ptr(offsets), total_M, N, K, _ptr(A), A.stride(0), _ptr(sA), sA.stride(0),
            _ptr(B), _ptr(sB), _ptr(out), code, out.stride(0), _stream(stream))
        _lib.check("fp8_block_gemm_grouped_tiled", st)
        return out
    st = lib.fp8_block_gemm_grouped(
        G, _ptr(offsets), total_M, N, K, _ptr(A), A.stride(0), _ptr(sA), sA.stride(0),
        _ptr(B), B.stride(1), _ptr(sB), _ptr(out), code, out.stride(0), _stream(stream))
    _lib.check("fp8_block_gemm_grouped", st)
    return out


def amax_history_update(hist: torch.Tensor, amax: torch.Tensor, *, decay: float = 0.9,
                        init: bool = False, scales_out=None, stream=None):
    """In-place h <- decay * h + (1 - decay) * amax (or h <- amax when init)."""
    lib = _lib.load_library()
    for n, t in (("hist", hist), ("amax", amax)):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{n}: contiguous float32 device tensor required")
    st = lib.fp8_amax_history_update(_ptr(hist), _ptr(amax), hist.numel(), float(decay),
                                     1 if init else 0, _ptr(scales_out), _stream(stream))
    _lib.check("fp8_amax_history_update", st)
    return hist


def cast_e4m3(x: torch.Tensor, *, out=None, stream=None):
    """Saturating round-to-nearest-even FP32 -> E4M3 codes (uint8)."""
    lib = _lib.load_library()
    if x.dtype != torch.float32 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x: contiguous float32 device tensor required")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    st = lib.fp8_cast_e4m3(_ptr(x), x.numel(), _ptr(out), _stream(stream))
    _lib.check("fp8_cast_e4m3", st)
    return out


def message_bytes(H: int) -> int:
    """Bytes of one token message: H codes + H/128 FP32 scales."""
    return H + H // 32


def pack_tokens(x: torch.Tensor, src_rows=None, *, T=None, stride=None, out=None, stream=None):
    """Quantize tokens x [rows][H] BF16 into messages uint8 [T][stride].

    src_rows: optional int32 device tensor [T]; message t carries row
    src_rows[t] (dispatch order).  Default: every row in order.
    stride defaults to round_up(H + H/32, 16).
    """
    lib = _lib.load_library()
    _check_2d("x", x, _BF16)
    rows, H = x.shape
    if src_rows is not None:
        if src_rows.dtype != torch.int32 or src_rows.dim() != 1 or not src_rows.is_contiguous():
            raise ValueError("src_rows: contiguous 1-D int32 device tensor required")
        T = src_rows.numel()
    elif T is None:
        T = rows
    stride = round_up(message_bytes(H), 16) if stride is None else stride
    if out is None:
        out = torch.empty((T, stride), dtype=torch.uint8, device=x.device)
    st = lib.fp8_pack_tokens(_ptr(x), rows, H, x.stride(0), _ptr(src_rows), T, _ptr(out),
                             out.stride(0), _stream(stream))
    _lib.check("fp8_pack_tokens", st)
    return out


def unpack_tokens(msg: torch.Tensor, H: int, *, stream=None):
    """Messages [T][stride] -> (q [T][H] uint8, scales [H/128][round_up(T, 4)] float32),
    the operand layout of quant_act_1x128(..., "row")."""
    lib = _lib.load_library()
    _check_2d("msg", msg, (torch.uint8,))
    T = msg.shape[0]
    q = torch.empty((T, H), dtype=torch.uint8, device=msg.device)
    s = torch.empty((H // 128, round_up(T, 4)), dtype=torch.float32, device=msg.device)
    st = lib.fp8_unpack_tokens(_ptr(msg), T, H, msg.stride(0), _ptr(q), q.stride(0), _ptr(s),
                               s.stride(0), _stream(stream))
    _lib.check("fp8_unpack_tokens", st)
    return q, s


def dequant_tokens(msg: torch.Tensor, H: int, *, stream=None):
    """Messages [T][stride] -> BF16 [T][H]: decode(q) * s rounded once to BF16."""
    lib = _lib.load_library()
    _check_2d("msg", msg, (torch.uint8,))
    T = msg.shape[0]
    y = torch.empty((T, H), dtype=torch.bfloat16, device=msg.device)
    st = lib.fp8_dequant_tokens(_ptr(msg), T, H, msg.stride(0), _ptr(y), y.stride(0), _stream(stream))
    _lib.check("fp8_dequant_tokens", st)
    return y


def gemm_promotion(A: torch.Tensor, B: torch.Tensor, promote_k: int, *, stream=None):
    """C [M][N] FP32 = A [M][K] . B [N][K]^T over E4M3 codes (unit scales), with
    the matrix unit's accumulator promoted to FP32 every promote_k values of K
    (32, 64 or a multiple of 128; >= K: one accumulator chain)."""
    lib = _lib.load_library()
    _check_2d("A", A, (torch.uint8,))
    _check_2d("B", B, (torch.uint8,))
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError(f"A {tuple(A.shape)} and B {tuple(B.shape)}: K differs")
    C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    st = lib.fp8_gemm_promotion(_ptr(A), M, K, A.stride(0), _ptr(B), N, B.stride(0), promote_k,
                                _ptr(C), C.stride(0), _stream(stream))
    _lib.check("fp8_gemm_promotion", st)
    return C


PROBE_MFMA_MODES = {"plain": 0, "scaled": 1, "fold": 2}


def probe_mfma(codes: torch.Tensor, workgroups: int, iters: int, mode: str = "plain", *, stream=None):
    """Measurement aid: `workgroups` x 4 waves each run 8 * iters independent
    FP8 MFMAs (65,536 FLOP each) on operands taken from `codes` (4096 uint8
    E4M3 codes: A from bytes 32 l.., B from 2048 + 32 l.. for lane l), with no
    memory traffic.  mode: "plain" (the GEMMs' MFMA), "scaled" (its
    block-scaled encoding, scales 2^0) or "fold" (plain MFMAs each followed by
    the 4 FP32 FMAs of the GEMMs' per-block fold).  Returns the per-lane
    checksums [workgroups * 256] float32."""
    lib = _lib.load_library()
    if codes.dtype != torch.uint8 or codes.numel() < 4096 or not codes.is_contiguous():
        raise ValueError("codes: a contiguous uint8 tensor of at least 4096 elements")
    if mode not in PROBE_MFMA_MODES:
        raise ValueError(f"mode: one of {sorted(PROBE_MFMA_MODES)}")
    out = torch.empty(workgroups * 256, dtype=torch.float32, device=codes.device)
    st = lib.fp8_probe_mfma(workgroups, iters, PROBE_MFMA_MODES[mode], _ptr(codes), _ptr(out), _stream(stream))
    _lib.check("fp8_probe_mfma", st)
    return out


def probe_recip_online(s: torch.Tensor, *, stream=None):
    """Verification aid: the quantizers' reciprocal of each online scale in s
    (float32 device tensor); returns r of the same shape."""
    lib = _lib.load_library()
    if s.dtype != torch.float32 or not s.is_contiguous():
        raise ValueError("s: a contiguous float32 tensor")
    r = torch.empty_like(s)
    st = lib.fp8_probe_recip_online(_ptr(s), _ptr(r), s.numel(), _stream(stream))
    _lib.check("fp8_probe_recip_online", st)
    return r


def probe_gemm_split(tiles: int, K: int, *, stream=None):
    """Measurement aid: (split_tiles, pieces) - how the persistent GEMM kernel
    schedules `tiles` output tiles of 128 x 256 with K-dimension K on `stream`:
    the number of leftover tiles cut along K and the pieces per such tile
    (0, 1: whole tiles only)."""
    lib = _lib.load_library()
    n = ctypes.c_int64(0)
    k = ctypes.c_int32(0)
    st = lib.fp8_probe_gemm_split(tiles, K, _stream(stream), ctypes.byref(n), ctypes.byref(k))
    _lib.check("fp8_probe_gemm_split", st)
    return n.value, k.value


def quant_act_tiles(x: torch.Tensor, tile: int = 128, rank: int = 1, *, sat_count=None, stream=None):
    """1 x tile quantization of x [rows][cols] BF16 with the clip value at the
    rank-th largest |x| of each tile (rank 1: the max).  Returns
    (q [rows][cols] uint8, scales [cols/tile][round_up(rows, 4)] float32).
    sat_count: optional one-element int32/uint32 device tensor, incremented."""
    lib = _lib.load_library()
    _check_2d("x", x, _BF16)
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((cols // tile, round_up(rows, 4)), dtype=torch.float32, device=x.device)
    st = lib.fp8_quant_act_tiles(_ptr(x), rows, cols, x.stride(0), tile, rank, _ptr(q), q.stride(0),
                                 _ptr(s), s.stride(0), _ptr(sat_count), _stream(stream))
    _lib.check("fp8_quant_act_tiles", st)
    return q, s
