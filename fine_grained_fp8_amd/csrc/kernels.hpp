// Host-side launchers of the HIP kernels (internal to libfp8bs.so).
// Arguments are already validated by api.cpp; each launcher only sizes the
// grid and enqueues on `stream`, returning the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                             const float* scales_in, float* amax_out, uint32_t* sat_count,
                             hipStream_t stream);

hipError_t launch_quant_cols(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                             float* amax_out, bool tiled, hipStream_t stream);

hipError_t launch_quant_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q_row, int64_t ldq_row, float* s_row, int64_t ld_s_row,
                             uint8_t* q_col, int64_t ldq_col, float* s_col, int64_t ld_s_col,
                             bool tiled, hipStream_t stream);

hipError_t launch_quant_weight(const uint16_t* w, int64_t rows, int64_t cols, int64_t ldw,
                               uint8_t* q, int64_t ldq, uint8_t* q_t, int64_t ldq_t,
                               float* scales, int64_t ld_s, bool tiled, hipStream_t stream);

hipError_t launch_history_update(float* hist, const float* amax, int64_t n, float decay, int init,
                                 float* scales_out, hipStream_t stream);

hipError_t launch_cast_e4m3(const float* x, int64_t n, uint8_t* q, hipStream_t stream);

hipError_t launch_pack_tokens(const uint16_t* x, int64_t x_rows, int64_t H, int64_t ldx,
                              const int32_t* src_rows, int64_t T, uint8_t* msg, int64_t stride,
                              hipStream_t stream);

hipError_t launch_unpack_tokens(const uint8_t* msg, int64_t T, int64_t H, int64_t stride,
                                uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                                hipStream_t stream);

hipError_t launch_dequant_tokens(const uint8_t* msg, int64_t T, int64_t H, int64_t stride,
                                 uint16_t* y, int64_t ldy, hipStream_t stream);

hipError_t launch_quant_tiles(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int tile,
                              int rank, uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                              uint32_t* sat_count, hipStream_t stream);

hipError_t launch_gemm_promotion(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                                 int64_t M, int64_t N, int64_t K, int64_t promote_k, float* C,
                                 int64_t ldc, hipStream_t stream);

hipError_t launch_mfma_probe(int64_t workgroups, int iters, int mode, const uint8_t* codes, float* out,
                             hipStream_t stream);
hipError_t launch_recip_online_probe(const float* s, float* r, int64_t n, hipStream_t stream);

enum GemmLayout { kFprop = 0, kDgrad = 1, kWgrad = 2, kDgradT = 3 };

struct GemmProblem {
  int layout;            // GemmLayout
  int64_t M, N, K;
  const uint8_t* A;      // token side (rows m), K-contiguous
  int64_t lda;
  const float* sA;       // [K/128][ld_sa]
  int64_t ld_sa;
  const uint8_t* B;      // weight side: [N][K] (FPROP, WGRAD, DGRAD_T) or [K][N] (DGRAD)
  int64_t ldb;
  const float* sB;
  int64_t ld_sb;
  void* C;
  int64_t ldc;
  int out_fp32;
  int b_tiled;           // B in the operand-tiled layout (FPROP, DGRAD_T, grouped; ldb == K)
  // grouped FPROP: groups > 0
  int groups;
  const int32_t* offsets;
  // split-K workspace of the persistent kernel (null: no split): ws_slots
  // partial tiles of kSplitTileFloats floats, then ws_slots counters that
  // are zero between launches
  float* ws_partial;
  uint32_t* ws_count;
  int64_t ws_slots;
};

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream);
// compute units of the current device (cached); 0 if unknown
int device_cus();
// workgroups of a persistent GEMM launch over `ids` tiles
int64_t persistent_grid(int64_t ids);

// ---- split-K tail of the persistent GEMM ----
// FP32 partial sums of one 128 x 256 output tile
constexpr int64_t kSplitTileFloats = 128 * 256;
constexpr int kMaxSplit = 16;
// Workspace bytes for `slots` pieces: the partial tiles, then the counters.
inline size_t split_workspace_bytes(int64_t slots) {
  return (size_t)slots * (size_t)kSplitTileFloats * 4u + (size_t)slots * 4u;
}

// pieces the static split workspace holds (one per CU up to this count)
constexpr int64_t kStaticSlots = 256;
// Point p's split workspace at the library's static array on the current
// device (found once per device; its counters cleared by a kernel on
// `stream` then).  Allocates nothing.
hipError_t attach_static_workspace(GemmProblem& p, hipStream_t stream);

// How a persistent launch of `grid` workgroups covers `tiles` output tiles
// of `kb` K blocks.  Whole rounds of one tile per workgroup come first
// (dp_tiles tiles).  When the leftover tiles would fill at most half of a
// last round, each of them is cut along K into `split` pieces of whole
// 4-block rounds, run by the workgroups that would otherwise idle; the
// fewest pieces that reach the shortest piece length are taken, since every
// extra piece adds a partial tile to the final sum.  split == 1: no split.
struct SplitPlan {
  int64_t dp_tiles;      // tiles run whole
  int64_t split_tiles;   // tiles run as `split` pieces each (tile ids dp_tiles..)
  int split;
  int rounds;            // 4-block rounds of K
};
__host__ __device__ inline SplitPlan split_plan(int64_t tiles, int64_t grid, int kb, int64_t slots) {
  SplitPlan s{tiles, 0, 1, (kb + 3) / 4};
  if (grid <= 0 || tiles <= grid || slots <= 0) return s;
  const int64_t left = tiles % grid;
  if (left == 0) return s;
  int64_t most = grid / left;
  if (most > kMaxSplit) most = kMaxSplit;
  if (most > s.rounds) most = s.rounds;
  if (most < 2) return s;
  const int64_t per = (s.rounds + most - 1) / most;      // rounds per piece at the most pieces
  const int64_t pieces = (s.rounds + per - 1) / per;     // the fewest pieces of that length
  if (pieces < 2 || left * pieces > slots) return s;
  s.dp_tiles = tiles - left;
  s.split_tiles = left;
  s.split = (int)pieces;
  return s;
}
// K blocks [lo, hi) of piece `piece` of a split tile
__host__ __device__ inline void split_range(const SplitPlan& s, int piece, int kb, int& lo, int& hi) {
  lo = 4 * (int)((int64_t)piece * s.rounds / s.split);
  hi = 4 * (int)((int64_t)(piece + 1) * s.rounds / s.split);
  if (hi > kb) hi = kb;
}

// Fprop with the 1x128 quantization of X fused in (BF16 X in).
struct FusedFpropProblem {
  int64_t M, N, K;
  const uint16_t* X;     // BF16 [M][ldx]
  int64_t ldx;
  const uint8_t* W;      // W_q [N][ldw]
  int64_t ldw;
  const float* sW;       // [N/128][ld_sw]
  int64_t ld_sw;
  void* C;
  int64_t ldc;
  int out_fp32;
  uint8_t* q_out;        // optional: the codes [M][ldq] and scales [K/128][ld_s]
  int64_t ldq;
  float* s_out;
  int64_t ld_s;
};
hipError_t launch_fused_quant_fprop(const FusedFpropProblem& p, hipStream_t stream);

}  // namespace fp8bs
