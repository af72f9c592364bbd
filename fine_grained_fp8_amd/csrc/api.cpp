// C ABI of libfp8bs.so: host-side validation, device check, dispatch to the
// kernel launchers.  Declarations and full contracts: include/fp8bs.h.
#include "fp8bs.h"
#include "fp8bs_probe.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "kernels.hpp"

namespace {

using fp8bs::GemmProblem;

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_device_kind[kMaxDevices];

fp8_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return FP8_ERR_DEVICE;
  }
  if (dev >= kMaxDevices) return FP8_ERR_DEVICE;
  int kind = g_device_kind[dev].load(std::memory_order_relaxed);
  if (kind == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return FP8_ERR_DEVICE;
    }
    kind = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_kind[dev].store(kind, std::memory_order_relaxed);
  }
  return kind == 1 ? FP8_OK : FP8_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// [lo, hi) byte range of a row-major matrix with `rows` rows of `row_bytes`
// at stride `ld_bytes`.
struct Range {
  uintptr_t lo, hi;
};
Range span(const void* p, int64_t rows, int64_t row_bytes, int64_t ld_bytes) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  if (rows <= 0 || row_bytes <= 0) return {b, b};
  return {b, b + static_cast<uintptr_t>((rows - 1) * ld_bytes + row_bytes)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// ---- split-K workspace of the persistent GEMM kernel ----
// One per (device, stream), allocated on the first GEMM call on that stream
// and kept until the process ends: partial tiles for one piece per
// workgroup of a full-device launch, and the per-tile counters (zeroed once
// on the stream; each launch leaves them zero).  Calls on one stream are
// ordered, so they share it safely; calls on different streams get
// different workspaces.  No workspace (and no split: the same results up to
// FP32 summation order, the whole-tile schedule) when the stream is being
// captured into a graph and has none yet, when the allocation fails, or when
// kMaxWorkspaces are held.
constexpr int kMaxWorkspaces = 64;
struct Workspace {
  int dev;
  hipStream_t stream;
  void* mem;
  int64_t slots;
};
std::mutex g_ws_mutex;
Workspace g_ws[kMaxWorkspaces];
int g_ws_used = 0;

// the workspace held for `stream` on the current device, or nullptr
const Workspace* find_workspace(int dev, hipStream_t stream) {
  for (int i = 0; i < g_ws_used; ++i)
    if (g_ws[i].dev == dev && g_ws[i].stream == stream) return &g_ws[i];
  return nullptr;
}

void attach_workspace(GemmProblem& p, hipStream_t stream) {
  p.ws_partial = nullptr;
  p.ws_count = nullptr;
  p.ws_slots = 0;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  const Workspace* w = find_workspace(dev, stream);
  if (w == nullptr) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) {
      (void)hipGetLastError();
      return;
    }
    const int64_t slots = fp8bs::device_cus();
    if (cap != hipStreamCaptureStatusNone || g_ws_used == kMaxWorkspaces || slots < 8) return;
    void* mem = nullptr;
    const size_t bytes = fp8bs::split_workspace_bytes(slots);
    if (hipMalloc(&mem, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return;
    }
    const size_t count_off = (size_t)slots * (size_t)fp8bs::kSplitTileFloats * 4u;
    if (hipMemsetAsync(static_cast<uint8_t*>(mem) + count_off, 0, (size_t)slots * 4u, stream) != hipSuccess) {
      (void)hipGetLastError();
      (void)hipFree(mem);
      return;
    }
    g_ws[g_ws_used] = Workspace{dev, stream, mem, slots};
    w = &g_ws[g_ws_used++];
  }
  p.ws_partial = static_cast<float*>(w->mem);
  p.ws_count = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(w->mem) +
                                           (size_t)w->slots * (size_t)fp8bs::kSplitTileFloats * 4u);
  p.ws_slots = w->slots;
}

fp8_status launched(hipError_t e) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return FP8_ERR_LAUNCH;
  }
  return FP8_OK;
}

}  // namespace

extern "C" {

int fp8_abi_version(void) { return FP8BS_ABI_VERSION; }

const char* fp8_status_string(fp8_status s) {
  switch (s) {
    case FP8_OK: return "ok";
    case FP8_ERR_NULL: return "a required pointer is NULL";
    case FP8_ERR_SHAPE: return "invalid shape (negative size, or a dimension is not a multiple of 128 where required)";
    case FP8_ERR_LD: return "leading dimension smaller than the row length";
    case FP8_ERR_ALIGN: return "pointer or row stride not 16-byte aligned";
    case FP8_ERR_UNSUPPORTED: return "unsupported enum value or argument combination";
    case FP8_ERR_DEVICE: return "no current HIP device, or the device is not gfx950";
    case FP8_ERR_LAUNCH: return "kernel launch failed";
    case FP8_ERR_ALIAS: return "an output buffer overlaps an input buffer";
  }
  return "unknown status";
}

fp8_status fp8_quant_act_1x128(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                               fp8_tile_dir dir, uint8_t* q, int64_t ldq,
                               float* scales, int64_t ld_s, const float* scales_in,
                               float* amax_out, uint32_t* sat_count, void* stream) {
  if (dir != FP8_TILE_ROW && dir != FP8_TILE_COL && dir != FP8_TILE_COL_TILED)
    return FP8_ERR_UNSUPPORTED;
  const bool tiled = dir == FP8_TILE_COL_TILED;
  if (tiled) {
    // dense operand tiles of the transposed codes: [cols][rows], cols % 128
    if (cols % 128 != 0) return FP8_ERR_SHAPE;
    if (ldq != rows) return FP8_ERR_LD;
    dir = FP8_TILE_COL;
  }
  if (rows < 0 || cols < 0) return FP8_ERR_SHAPE;
  if (dir == FP8_TILE_ROW && cols % 128 != 0) return FP8_ERR_SHAPE;
  if (dir == FP8_TILE_COL && rows % 128 != 0) return FP8_ERR_SHAPE;
  if (dir == FP8_TILE_COL && (scales_in || sat_count)) return FP8_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return FP8_OK;
  if (!x || !q) return FP8_ERR_NULL;
  if (!scales_in && !scales) return FP8_ERR_NULL;
  const int64_t out_rows = dir == FP8_TILE_ROW ? rows : cols;
  const int64_t out_cols = dir == FP8_TILE_ROW ? cols : rows;
  const int64_t s_rows = dir == FP8_TILE_ROW ? cols / 128 : rows / 128;
  const int64_t s_cols = dir == FP8_TILE_ROW ? rows : cols;
  if (ldx < cols || ldq < out_cols || ld_s < s_cols) return FP8_ERR_LD;
  if (!aligned16(x) || !aligned16(q) || (ldx * 2) % 16 != 0 || ldq % 16 != 0) return FP8_ERR_ALIGN;
  if ((scales && !aligned4(scales)) || (scales_in && !aligned4(scales_in)) ||
      (amax_out && !aligned4(amax_out)) || (sat_count && !aligned4(sat_count)))
    return FP8_ERR_ALIGN;
  const Range rx = span(x, rows, cols * 2, ldx * 2);
  const Range rq = span(q, out_rows, out_cols, ldq);
  const Range rs = span(scales ? (const void*)scales : (const void*)scales_in, s_rows, s_cols * 4, ld_s * 4);
  if (overlap(rq, rx)) return FP8_ERR_ALIAS;
  if (scales && (overlap(rs, rx) || overlap(rs, rq))) return FP8_ERR_ALIAS;
  if (amax_out) {
    const Range ra = span(amax_out, s_rows, s_cols * 4, ld_s * 4);
    if (overlap(ra, rx) || overlap(ra, rq) || (scales && overlap(ra, rs))) return FP8_ERR_ALIAS;
    if (scales_in && overlap(ra, span(scales_in, s_rows, s_cols * 4, ld_s * 4))) return FP8_ERR_ALIAS;
  }
  if (scales_in && overlap(rq, span(scales_in, s_rows, s_cols * 4, ld_s * 4))) return FP8_ERR_ALIAS;
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (dir == FP8_TILE_ROW)
    return launched(fp8bs::launch_quant_rows(xb, rows, cols, ldx, q, ldq, scales_in ? nullptr : scales,
                                             ld_s, scales_in, amax_out, sat_count, st));
  return launched(fp8bs::launch_quant_cols(xb, rows, cols, ldx, q, ldq, scales, ld_s, amax_out, tiled, st));
}

namespace {
fp8_status quant_dual_impl(const void* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* q_row,
                           int64_t ldq_row, float* s_row, int64_t ld_s_row, uint8_t* q_col,
                           int64_t ldq_col, float* s_col, int64_t ld_s_col, bool tiled, void* stream) {
  if (rows < 0 || cols < 0 || rows % 128 != 0 || cols % 128 != 0) return FP8_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8_OK;
  if (!x || !q_row || !s_row || !q_col || !s_col) return FP8_ERR_NULL;
  if (ldx < cols || ldq_row < cols || ld_s_row < rows || ldq_col < rows || ld_s_col < cols)
    return FP8_ERR_LD;
  if (!aligned16(x) || !aligned16(q_row) || !aligned16(q_col) || (ldx * 2) % 16 != 0 ||
      ldq_row % 16 != 0 || ldq_col % 16 != 0 || !aligned4(s_row) || !aligned4(s_col))
    return FP8_ERR_ALIGN;
  const Range rx = span(x, rows, cols * 2, ldx * 2);
  const Range rqr = span(q_row, rows, cols, ldq_row);
  const Range rsr = span(s_row, cols / 128, rows * 4, ld_s_row * 4);
  const Range rqc = span(q_col, cols, rows, ldq_col);
  const Range rsc = span(s_col, rows / 128, cols * 4, ld_s_col * 4);
  const Range outs[4] = {rqr, rsr, rqc, rsc};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], rx)) return FP8_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return FP8_ERR_ALIAS;
  }
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  return launched(fp8bs::launch_quant_dual(static_cast<const uint16_t*>(x), rows, cols, ldx, q_row,
                                           ldq_row, s_row, ld_s_row, q_col, ldq_col, s_col, ld_s_col,
                                           tiled, reinterpret_cast<hipStream_t>(stream)));
}
}  // namespace

fp8_status fp8_quant_act_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                              uint8_t* q_row, int64_t ldq_row, float* s_row, int64_t ld_s_row,
                              uint8_t* q_col, int64_t ldq_col, float* s_col, int64_t ld_s_col,
                              void* stream) {
  return quant_dual_impl(x, rows, cols, ldx, q_row, ldq_row, s_row, ld_s_row, q_col, ldq_col, s_col,
                         ld_s_col, false, stream);
}

fp8_status fp8_quant_act_dual_tiled(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                    uint8_t* q_row, int64_t ldq_row, float* s_row, int64_t ld_s_row,
                                    uint8_t* q_col_tiled, float* s_col, int64_t ld_s_col,
                                    void* stream) {
  return quant_dual_impl(x, rows, cols, ldx, q_row, ldq_row, s_row, ld_s_row, q_col_tiled, rows, s_col,
                         ld_s_col, true, stream);
}

fp8_status fp8_pack_tokens(const void* x, int64_t x_rows, int64_t H, int64_t ldx,
                           const int32_t* src_rows, int64_t T, uint8_t* msg, int64_t stride,
                           void* stream) {
  if (x_rows < 0 || H < 0 || T < 0 || H % 128 != 0) return FP8_ERR_SHAPE;
  if (!src_rows && T > x_rows) return FP8_ERR_SHAPE;
  if (T == 0 || H == 0) return FP8_OK;
  if (!msg || (!x && x_rows > 0)) return FP8_ERR_NULL;
  if (ldx < H || stride < H + H / 32) return FP8_ERR_LD;
  if (!aligned16(x) || !aligned16(msg) || (ldx * 2) % 16 != 0 || stride % 16 != 0 ||
      !aligned4(src_rows))
    return FP8_ERR_ALIGN;
  const Range rm = span(msg, T, H + H / 32, stride);
  if (overlap(rm, span(x, x_rows, H * 2, ldx * 2))) return FP8_ERR_ALIAS;
  if (src_rows && overlap(rm, span(src_rows, 1, T * 4, T * 4))) return FP8_ERR_ALIAS;
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  return launched(fp8bs::launch_pack_tokens(static_cast<const uint16_t*>(x), x_rows, H, ldx, src_rows,
                                            T, msg, stride, reinterpret_cast<hipStream_t>(stream)));
}

fp8_status fp8_unpack_tokens(const uint8_t* msg, int64_t T, int64_t H, int64_t stride, uint8_t* q,
                             int64_t ldq, float* scales, int64_t ld_s, void* stream) {
  if (T < 0 || H < 0 || H % 128 != 0) return FP8_ERR_SHAPE;
  if (T == 0 || H == 0) return FP8_OK;
  if (!msg || !q || !scales) return FP8_ERR_NULL;
  if (stride < H + H / 32 || ldq < H || ld_s < T) return FP8_ERR_LD;
  if (!aligned16(msg) || !aligned16(q) || stride % 16 != 0 || ldq % 16 != 0 || !aligned4(scales))
    return FP8_ERR_ALIGN;
  const Range rm = span(msg, T, H + H / 32, stride);
  const Range rq = span(q, T, H, ldq);
  const Range rs = span(scales, H / 128, T * 4, ld_s * 4);
  if (overlap(rq, rm) || overlap(rs, rm) || overlap(rq, rs)) return FP8_ERR_ALIAS;
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  return launched(fp8bs::launch_unpack_tokens(msg, T, H, stride, q, ldq, scales, ld_s,
                                              reinterpret_cast<hipStream_t>(stream)));
}

fp8_status fp8_dequant_tokens(const uint8_t* msg, int64_t T, int64_t H, int64_t stride, void* y,
                              int64_t ldy, void* stream) {
  if (T < 0 || H < 0 || H % 128 != 0) return FP8_ERR_SHAPE;
  if (T == 0 || H == 0) return FP8_OK;
  if (!msg || !y) return FP8_ERR_NULL;
  if (stride < H + H / 32 || ldy < H) return FP8_ERR_LD;
  if (!aligned16(msg) || !aligned16(y) || stride % 16 != 0 || (ldy * 2) % 16 != 0)
    return FP8_ERR_ALIGN;
  if (overlap(span(y, T, H * 2, ldy * 2), span(msg, T, H + H / 32, stride))) return FP8_ERR_ALIAS;
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  return launched(fp8bs::launch_dequant_tokens(msg, T, H, stride, static_cast<uint16_t*>(y), ldy,
                                               reinterpret_cast<hipStream_t>(stream)));
}

fp8_status fp8_quant_act_tiles(const void* x, int64_t rows, int64_t cols, int64_t ldx, int32_t tile,
                               int32_t rank, uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                               uint32_t* sat_count, void* stream) {
  if (!(tile == 32 || tile == 64 || tile == 128 || tile == 256 || tile == 512 || tile == 1024) ||
      rank < 1 || rank > 8)
    return FP8_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || cols % tile != 0) return FP8_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8_OK;
  if (!x || !q || !scales) return FP8_ERR_NULL;
  if (ldx < cols || ldq < cols || ld_s < rows) return FP8_ERR_LD;
  if (!aligned16(x) || !aligned16(q) || (ldx * 2) % 16 != 0 || ldq % 16 != 0 || !aligned4(scales) ||
      !aligned4(sat_count))
    return FP8_ERR_ALIGN;
  const Range rx = span(x, rows, cols * 2, ldx * 2);
  const Range rq = span(q, rows, cols, ldq);
  const Range rs = span(scales, cols / tile, rows * 4, ld_s * 4);
  if (overlap(rq, rx) || overlap(rs, rx) || overlap(rq, rs)) return FP8_ERR_ALIAS;
  if (sat_count) {
    const Range rc = span(sat_count, 1, 4, 4);
    if (overlap(rc, rx) || overlap(rc, rq) || overlap(rc, rs)) return FP8_ERR_ALIAS;
  }
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  return launched(fp8bs::launch_quant_tiles(static_cast<const uint16_t*>(x), rows, cols, ldx, tile, rank,
                                            q, ldq, scales, ld_s, sat_count,
                                            reinterpret_cast<hipStream_t>(stream)));
}

fp8_status fp8_probe_mfma(int64_t workgroups, int32_t iters, int32_t mode, const uint8_t* codes,
                          float* out, void* stream) {
  if (workgroups < 1 || workgroups > (int64_t{1} << 20) || iters < 1) return FP8_ERR_SHAPE;
  if (mode != FP8_PROBE_MFMA_PLAIN && mode != FP8_PROBE_MFMA_SCALED && mode != FP8_PROBE_MFMA_FOLD)
    return FP8_ERR_SHAPE;
  if (!codes || !out) return FP8_ERR_NULL;
  if (!aligned16(codes) || !aligned4(out)) return FP8_ERR_ALIGN;
  if (overlap(span(codes, 1, 4096, 0), span(out, 1, workgroups * 256 * 4, 0))) return FP8_ERR_ALIAS;
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  return launched(fp8bs::launch_mfma_probe(workgroups, iters, mode, codes, out,
                                           reinterpret_cast<hipStream_t>(stream)));
}

fp8_status fp8_probe_gemm_split(int64_t tiles, int64_t K, void* stream, int64_t* split_tiles, int32_t* pieces) {
  if (tiles < 0 || K <= 0 || K % 128 != 0) return FP8_ERR_SHAPE;
  if (!split_tiles || !pieces) return FP8_ERR_NULL;
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  int d = -1;
  if (hipGetDevice(&d) != hipSuccess) {
    (void)hipGetLastError();
    return FP8_ERR_DEVICE;
  }
  int64_t slots = 0;
  {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    const Workspace* w = find_workspace(d, reinterpret_cast<hipStream_t>(stream));
    if (w) slots = w->slots;
  }
  const int64_t kb = K / 128;
  const fp8bs::SplitPlan plan =
      fp8bs::split_plan(tiles, fp8bs::persistent_grid(tiles), kb > (1 << 30) ? (1 << 30) : (int)kb, slots);
  *split_tiles = plan.split_tiles;
  *pieces = plan.split;
  return FP8_OK;
}

fp8_status fp8_probe_recip_online(const float* s, float* r, int64_t n, void* stream) {
  if (n < 0 || n > (int64_t{1} << 30)) return FP8_ERR_SHAPE;
  if (n == 0) return FP8_OK;
  if (!s || !r) return FP8_ERR_NULL;
  if (!aligned4(s) || !aligned4(r)) return FP8_ERR_ALIGN;
  if (overlap(span(s, 1, n * 4, 0), span(r, 1, n * 4, 0))) return FP8_ERR_ALIAS;
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  return launched(fp8bs::launch_recip_online_probe(s, r, n, reinterpret_cast<hipStream_t>(stream)));
}

fp8_status fp8_gemm_promotion(const uint8_t* A, int64_t M, int64_t K, int64_t lda, const uint8_t* B,
                              int64_t N, int64_t ldb, int64_t promote_k, float* C, int64_t ldc,
                              void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0) return FP8_ERR_SHAPE;
  if (!(promote_k == 32 || promote_k == 64 || (promote_k >= 128 && promote_k % 128 == 0)))
    return FP8_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return FP8_OK;
  if (!C || (K > 0 && (!A || !B))) return FP8_ERR_NULL;
  if (lda < K || ldb < K || ldc < N) return FP8_ERR_LD;
  if (!aligned16(A) || !aligned16(B) || lda % 16 != 0 || ldb % 16 != 0 || !aligned4(C))
    return FP8_ERR_ALIGN;
  const Range rc = span(C, M, N * 4, ldc * 4);
  if (overlap(rc, span(A, M, K, lda)) || overlap(rc, span(B, N, K, ldb))) return FP8_ERR_ALIAS;
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  return launched(fp8bs::launch_gemm_promotion(A, lda, B, ldb, M, N, K, promote_k, C, ldc,
                                               reinterpret_cast<hipStream_t>(stream)));
}

namespace {
fp8_status quant_weight_impl(const void* w, int64_t rows, int64_t cols, int64_t ldw, uint8_t* q,
                             int64_t ldq, uint8_t* q_t, int64_t ldq_t, float* scales, int64_t ld_s,
                             bool tiled, void* stream) {
  if (rows < 0 || cols < 0 || rows % 128 != 0 || cols % 128 != 0) return FP8_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP8_OK;
  if (!w || !q || !scales) return FP8_ERR_NULL;
  if (ldw < cols || ldq < cols || ld_s < cols / 128 || (q_t && ldq_t < rows)) return FP8_ERR_LD;
  if (!aligned16(w) || !aligned16(q) || (ldw * 2) % 16 != 0 || ldq % 16 != 0 || !aligned4(scales))
    return FP8_ERR_ALIGN;
  if (q_t && (!aligned16(q_t) || ldq_t % 16 != 0)) return FP8_ERR_ALIGN;
  const Range rw = span(w, rows, cols * 2, ldw * 2);
  const Range rq = span(q, rows, cols, ldq);
  const Range rs = span(scales, rows / 128, (cols / 128) * 4, ld_s * 4);
  if (overlap(rq, rw) || overlap(rs, rw) || overlap(rs, rq)) return FP8_ERR_ALIAS;
  if (q_t) {
    const Range rt = span(q_t, cols, rows, ldq_t);
    if (overlap(rt, rw) || overlap(rt, rq) || overlap(rt, rs)) return FP8_ERR_ALIAS;
  }
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  return launched(fp8bs::launch_quant_weight(static_cast<const uint16_t*>(w), rows, cols, ldw, q, ldq,
                                             q_t, ldq_t, scales, ld_s, tiled,
                                             reinterpret_cast<hipStream_t>(stream)));
}
}  // namespace

fp8_status fp8_quant_weight_128x128(const void* w, int64_t rows, int64_t cols, int64_t ldw,
                                    uint8_t* q, int64_t ldq, uint8_t* q_t, int64_t ldq_t,
                                    float* scales, int64_t ld_s, void* stream) {
  return quant_weight_impl(w, rows, cols, ldw, q, ldq, q_t, ldq_t, scales, ld_s, false, stream);
}

fp8_status fp8_quant_weight_128x128_tiled(const void* w, int64_t rows, int64_t cols, int64_t ldw,
                                          uint8_t* q_tiled, uint8_t* q_t_tiled, float* scales,
                                          int64_t ld_s, void* stream) {
  // the tiled arrays are dense: rows * cols bytes each
  return quant_weight_impl(w, rows, cols, ldw, q_tiled, cols, q_t_tiled, rows, scales, ld_s, true,
                           stream);
}

static fp8_status validate_gemm_common(int64_t M, int64_t N, int64_t K, const uint8_t* A,
                                       int64_t lda, const float* sA, int64_t ld_sa,
                                       const uint8_t* B, const float* sB, void* C,
                                       fp8_out_dtype c_dtype, int64_t ldc) {
  if (c_dtype != FP8_OUT_BF16 && c_dtype != FP8_OUT_FP32) return FP8_ERR_UNSUPPORTED;
  if (M < 0 || N <= 0 || K <= 0 || K % 128 != 0) return FP8_ERR_SHAPE;
  if (M == 0) return FP8_OK;
  if (!A || !sA || !B || !sB || !C) return FP8_ERR_NULL;
  if (lda < K || ld_sa < M || ldc < N) return FP8_ERR_LD;
  // the kernels address one 256-row tile, and a scale table's K blocks, with
  // 32-bit byte offsets
  if (lda > (int64_t{1} << 23)) return FP8_ERR_UNSUPPORTED;
  if ((K / 128) * ld_sa * 4 >= (int64_t{1} << 31)) return FP8_ERR_UNSUPPORTED;
  const int64_t esz = c_dtype == FP8_OUT_FP32 ? 4 : 2;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C) || lda % 16 != 0 || (ldc * esz) % 16 != 0 ||
      !aligned4(sA) || !aligned4(sB))
    return FP8_ERR_ALIGN;
  return FP8_OK;
}

namespace {
fp8_status block_gemm_impl(fp8_gemm_layout layout, int64_t M, int64_t N, int64_t K,
                           const uint8_t* A, int64_t lda, const float* sA, int64_t ld_sa,
                           const uint8_t* B, int64_t ldb, const float* sB, int64_t ld_sb,
                           void* C, fp8_out_dtype c_dtype, int64_t ldc, void* stream, bool noalloc) {
  if (layout != FP8_LAYOUT_FPROP && layout != FP8_LAYOUT_DGRAD && layout != FP8_LAYOUT_WGRAD &&
      layout != FP8_LAYOUT_DGRAD_T && layout != FP8_LAYOUT_FPROP_TILED &&
      layout != FP8_LAYOUT_DGRAD_T_TILED && layout != FP8_LAYOUT_WGRAD_TILED)
    return FP8_ERR_UNSUPPORTED;
  const bool tiled = layout == FP8_LAYOUT_FPROP_TILED || layout == FP8_LAYOUT_DGRAD_T_TILED ||
                     layout == FP8_LAYOUT_WGRAD_TILED;
  if (tiled && N % 128 != 0) return FP8_ERR_SHAPE;
  if (layout == FP8_LAYOUT_FPROP_TILED) layout = FP8_LAYOUT_FPROP;
  if (layout == FP8_LAYOUT_DGRAD_T_TILED) layout = FP8_LAYOUT_DGRAD_T;
  if (layout == FP8_LAYOUT_WGRAD_TILED) layout = FP8_LAYOUT_WGRAD;
  fp8_status st = validate_gemm_common(M, N, K, A, lda, sA, ld_sa, B, sB, C, c_dtype, ldc);
  if (st != FP8_OK || M == 0) return st;
  if (layout != FP8_LAYOUT_WGRAD && N % 128 != 0) return FP8_ERR_SHAPE;
  // the kernels number output tiles in 32 bits
  if (((M + 127) / 128) * ((N + 255) / 256) >= (int64_t{1} << 31)) return FP8_ERR_UNSUPPORTED;
  int64_t b_rows, b_cols, sb_rows, sb_cols;
  switch (layout) {
    case FP8_LAYOUT_FPROP: b_rows = N; b_cols = K; sb_rows = N / 128; sb_cols = K / 128; break;
    case FP8_LAYOUT_DGRAD: b_rows = K; b_cols = N; sb_rows = K / 128; sb_cols = N / 128; break;
    case FP8_LAYOUT_DGRAD_T: b_rows = N; b_cols = K; sb_rows = K / 128; sb_cols = N / 128; break;
    default: b_rows = N; b_cols = K; sb_rows = K / 128; sb_cols = N; break;
  }
  if (ldb < b_cols || ld_sb < sb_cols) return FP8_ERR_LD;
  if (tiled && ldb != K) return FP8_ERR_LD;       // dense tiles: the row "stride" is K
  if (ldb % 16 != 0) return FP8_ERR_ALIGN;
  if (ldb > (int64_t{1} << 23)) return FP8_ERR_UNSUPPORTED;
  // the scale tables are read through buffers whose byte range is 32-bit
  if (sb_rows * ld_sb * 4 >= (int64_t{1} << 31)) return FP8_ERR_UNSUPPORTED;
  if (layout == FP8_LAYOUT_DGRAD && K * ldb >= (int64_t{1} << 31)) return FP8_ERR_UNSUPPORTED;
  const int64_t esz = c_dtype == FP8_OUT_FP32 ? 4 : 2;
  const Range rc = span(C, M, N * esz, ldc * esz);
  if (overlap(rc, span(A, M, K, lda)) || overlap(rc, span(B, b_rows, b_cols, ldb)) ||
      overlap(rc, span(sA, K / 128, M * 4, ld_sa * 4)) ||
      overlap(rc, span(sB, sb_rows, sb_cols * 4, ld_sb * 4)))
    return FP8_ERR_ALIAS;
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  GemmProblem p{};
  p.layout = static_cast<int>(layout);
  p.M = M; p.N = N; p.K = K;
  p.A = A; p.lda = lda; p.sA = sA; p.ld_sa = ld_sa;
  p.B = B; p.ldb = ldb; p.sB = sB; p.ld_sb = ld_sb;
  p.C = C; p.ldc = ldc; p.out_fp32 = c_dtype == FP8_OUT_FP32;
  p.b_tiled = tiled ? 1 : 0;
  p.groups = 0; p.offsets = nullptr;
  if (noalloc) {
    // the static workspace holds one piece per CU of up to kStaticSlots CUs
    if (fp8bs::device_cus() > fp8bs::kStaticSlots) return FP8_ERR_UNSUPPORTED;
    if (fp8bs::attach_static_workspace(p, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) {
      (void)hipGetLastError();
      return FP8_ERR_LAUNCH;
    }
  } else {
    attach_workspace(p, reinterpret_cast<hipStream_t>(stream));
  }
  return launched(fp8bs::launch_gemm(p, reinterpret_cast<hipStream_t>(stream)));
}
}  // namespace

fp8_status fp8_block_gemm(fp8_gemm_layout layout, int64_t M, int64_t N, int64_t K,
                          const uint8_t* A, int64_t lda, const float* sA, int64_t ld_sa,
                          const uint8_t* B, int64_t ldb, const float* sB, int64_t ld_sb,
                          void* C, fp8_out_dtype c_dtype, int64_t ldc, void* stream) {
  return block_gemm_impl(layout, M, N, K, A, lda, sA, ld_sa, B, ldb, sB, ld_sb, C, c_dtype, ldc, stream, false);
}

fp8_status fp8_block_gemm_noalloc(fp8_gemm_layout layout, int64_t M, int64_t N, int64_t K,
                                  const uint8_t* A, int64_t lda, const float* sA, int64_t ld_sa,
                                  const uint8_t* B, int64_t ldb, const float* sB, int64_t ld_sb,
                                  void* C, fp8_out_dtype c_dtype, int64_t ldc, void* stream) {
  return block_gemm_impl(layout, M, N, K, A, lda, sA, ld_sa, B, ldb, sB, ld_sb, C, c_dtype, ldc, stream, true);
}

fp8_status fp8_block_gemm_fused_quant(int64_t M, int64_t N, int64_t K, const void* x, int64_t ldx,
                                     const uint8_t* W, int64_t ldw, const float* sW, int64_t ld_sw,
                                     void* C, fp8_out_dtype c_dtype, int64_t ldc, uint8_t* q_out,
                                     int64_t ldq, float* s_out, int64_t ld_s, void* stream) {
  if (c_dtype != FP8_OUT_BF16 && c_dtype != FP8_OUT_FP32) return FP8_ERR_UNSUPPORTED;
  if (M < 0 || N <= 0 || K <= 0 || K % 128 != 0 || N % 128 != 0) return FP8_ERR_SHAPE;
  if (M == 0) return FP8_OK;
  if (!x || !W || !sW || !C) return FP8_ERR_NULL;
  if ((q_out == nullptr) != (s_out == nullptr)) return FP8_ERR_NULL;
  if (ldx < K || ldw < K || ld_sw < K / 128 || ldc < N) return FP8_ERR_LD;
  if (q_out && (ldq < K || ld_s < M)) return FP8_ERR_LD;
  const int64_t esz = c_dtype == FP8_OUT_FP32 ? 4 : 2;
  if (!aligned16(x) || ldx % 8 != 0 || !aligned16(W) || ldw % 16 != 0 || !aligned16(C) ||
      (ldc * esz) % 16 != 0 || !aligned4(sW))
    return FP8_ERR_ALIGN;
  if (q_out && (!aligned16(q_out) || ldq % 16 != 0 || !aligned4(s_out))) return FP8_ERR_ALIGN;
  // one 128-row tile of X or W, and the weight-scale row, within 32-bit byte offsets
  if (ldx > (int64_t{1} << 22) || ldw > (int64_t{1} << 23)) return FP8_ERR_UNSUPPORTED;
  const Range rc = span(C, M, N * esz, ldc * esz);
  if (overlap(rc, span(x, M, K * 2, ldx * 2)) || overlap(rc, span(W, N, K, ldw)) ||
      overlap(rc, span(sW, N / 128, (K / 128) * 4, ld_sw * 4)))
    return FP8_ERR_ALIAS;
  if (q_out) {
    const Range rq = span(q_out, M, K, ldq), rs = span(s_out, K / 128, M * 4, ld_s * 4);
    if (overlap(rq, rc) || overlap(rs, rc) || overlap(rq, rs) || overlap(rq, span(x, M, K * 2, ldx * 2)) ||
        overlap(rs, span(x, M, K * 2, ldx * 2)))
      return FP8_ERR_ALIAS;
  }
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  fp8bs::FusedFpropProblem p{};
  p.M = M; p.N = N; p.K = K;
  p.X = static_cast<const uint16_t*>(x); p.ldx = ldx;
  p.W = W; p.ldw = ldw; p.sW = sW; p.ld_sw = ld_sw;
  p.C = C; p.ldc = ldc; p.out_fp32 = c_dtype == FP8_OUT_FP32;
  p.q_out = q_out; p.ldq = ldq; p.s_out = s_out; p.ld_s = ld_s;
  return launched(fp8bs::launch_fused_quant_fprop(p, reinterpret_cast<hipStream_t>(stream)));
}

namespace {
fp8_status grouped_impl(int32_t groups, const int32_t* offsets_dev, int64_t total_M, int64_t N,
                        int64_t K, const uint8_t* A, int64_t lda, const float* sA, int64_t ld_sa,
                        const uint8_t* B, int64_t ldb, const float* sB, void* C,
                        fp8_out_dtype c_dtype, int64_t ldc, bool tiled, void* stream) {
  if (groups <= 0) return FP8_ERR_SHAPE;
  fp8_status st = validate_gemm_common(total_M, N, K, A, lda, sA, ld_sa, B, sB, C, c_dtype, ldc);
  if (st != FP8_OK || total_M == 0) return st;
  if (!offsets_dev) return FP8_ERR_NULL;
  // tile count bound (every group may end in a ragged tile), numbered in 32 bits
  if (((total_M + 127) / 128 + groups) * ((N + 255) / 256) >= (int64_t{1} << 31)) return FP8_ERR_UNSUPPORTED;
  if (!aligned4(offsets_dev)) return FP8_ERR_ALIGN;
  if (N % 128 != 0) return FP8_ERR_SHAPE;
  if (ldb < K || (tiled && ldb != K)) return FP8_ERR_LD;
  if (ldb % 16 != 0) return FP8_ERR_ALIGN;
  if (ldb > (int64_t{1} << 23)) return FP8_ERR_UNSUPPORTED;
  if ((N / 128) * (K / 128) >= (int64_t{1} << 29)) return FP8_ERR_UNSUPPORTED;
  const int64_t esz = c_dtype == FP8_OUT_FP32 ? 4 : 2;
  const Range rc = span(C, total_M, N * esz, ldc * esz);
  if (overlap(rc, span(A, total_M, K, lda)) ||
      overlap(rc, span(B, static_cast<int64_t>(groups) * N, K, ldb)) ||
      overlap(rc, span(sA, K / 128, total_M * 4, ld_sa * 4)) ||
      overlap(rc, span(sB, 1, static_cast<int64_t>(groups) * (N / 128) * (K / 128) * 4, 0)) ||
      overlap(rc, span(offsets_dev, 1, (static_cast<int64_t>(groups) + 1) * 4, 0)))
    return FP8_ERR_ALIAS;
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  GemmProblem p{};
  p.layout = FP8_LAYOUT_FPROP;
  p.M = total_M; p.N = N; p.K = K;
  p.A = A; p.lda = lda; p.sA = sA; p.ld_sa = ld_sa;
  p.B = B; p.ldb = ldb; p.sB = sB; p.ld_sb = K / 128;
  p.C = C; p.ldc = ldc; p.out_fp32 = c_dtype == FP8_OUT_FP32;
  p.b_tiled = tiled ? 1 : 0;
  p.groups = groups; p.offsets = offsets_dev;
  attach_workspace(p, reinterpret_cast<hipStream_t>(stream));
  return launched(fp8bs::launch_gemm(p, reinterpret_cast<hipStream_t>(stream)));
}
}  // namespace

fp8_status fp8_block_gemm_grouped(int32_t groups, const int32_t* offsets_dev, int64_t total_M,
                                  int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                  const float* sA, int64_t ld_sa, const uint8_t* B, int64_t ldb,
                                  const float* sB, void* C, fp8_out_dtype c_dtype, int64_t ldc,
                                  void* stream) {
  return grouped_impl(groups, offsets_dev, total_M, N, K, A, lda, sA, ld_sa, B, ldb, sB, C, c_dtype,
                      ldc, false, stream);
}

fp8_status fp8_block_gemm_grouped_tiled(int32_t groups, const int32_t* offsets_dev, int64_t total_M,
                                        int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                        const float* sA, int64_t ld_sa, const uint8_t* B,
                                        const float* sB, void* C, fp8_out_dtype c_dtype,
                                        int64_t ldc, void* stream) {
  return grouped_impl(groups, offsets_dev, total_M, N, K, A, lda, sA, ld_sa, B, K, sB, C, c_dtype,
                      ldc, true, stream);
}

fp8_status fp8_amax_history_update(float* hist, const float* amax, int64_t n, float decay,
                                   int init, float* scales_out, void* stream) {
  if (n < 0) return FP8_ERR_SHAPE;
  if (n == 0) return FP8_OK;
  if (!hist || !amax) return FP8_ERR_NULL;
  if (!aligned4(hist) || !aligned4(amax) || (scales_out && !aligned4(scales_out))) return FP8_ERR_ALIGN;
  const Range rh = span(hist, 1, n * 4, 0);
  if (overlap(rh, span(amax, 1, n * 4, 0))) return FP8_ERR_ALIAS;
  if (scales_out && (overlap(span(scales_out, 1, n * 4, 0), rh) ||
                     overlap(span(scales_out, 1, n * 4, 0), span(amax, 1, n * 4, 0))))
    return FP8_ERR_ALIAS;
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  return launched(fp8bs::launch_history_update(hist, amax, n, decay, init, scales_out,
                                               reinterpret_cast<hipStream_t>(stream)));
}

fp8_status fp8_cast_e4m3(const float* x, int64_t n, uint8_t* q, void* stream) {
  if (n < 0) return FP8_ERR_SHAPE;
  if (n == 0) return FP8_OK;
  if (!x || !q) return FP8_ERR_NULL;
  if (!aligned4(x)) return FP8_ERR_ALIGN;
  if (overlap(span(x, 1, n * 4, 0), span(q, 1, n, 0))) return FP8_ERR_ALIAS;
  const fp8_status dev = check_device();
  if (dev != FP8_OK) return dev;
  return launched(fp8bs::launch_cast_e4m3(x, n, q, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
