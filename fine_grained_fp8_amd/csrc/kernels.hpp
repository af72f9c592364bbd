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
};

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream);

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
