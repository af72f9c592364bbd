// FP8 GEMM with a chosen promotion interval: how far the matrix unit's own
// accumulator may carry a sum before it is moved into an FP32 running sum.
//
// Sources: "Introduction to LLM Quantization" section 3 (tensor cores keep
// FP8 GEMM sums with limited precision; partial sums are promoted to FP32 at
// a fixed interval); "FP8 Mixed Precision: DeepSeek-V3 Training
// Architecture" section 3 (partial products accumulated in FP32 registers).
//
// C[m][n] = sum_k A[m][k] B[n][k] over E4M3 codes (unit scales), FP32 out.
//  - promote_k a multiple of 128: one v_mfma_f32_16x16x128_f8f6f4 per
//    128-wide K block with the MFMA accumulator carried from block to block
//    (the MFMA's C input) for promote_k / 128 blocks, then added to the FP32
//    running sum and cleared.  promote_k = 128 is the method's interval and
//    gives bit for bit the block GEMM's result with unit scales; promote_k
//    >= K is one accumulator chain over all of K.
//  - promote_k 32 or 64: every 128-wide block is split into sub-blocks whose
//    MFMA partials (operands outside the sub-block zeroed) are each added to
//    the running sum.
// One wave computes one 16x16 output tile; operands are read straight from
// memory in the byte order of the block GEMM's direct kernel (lane group g:
// bytes 16g.. and 64+16g.. of the K block), so the MFMA sees the same k
// grouping.  Not tuned for speed: it exists to measure accumulation error.
#include "device.hpp"
#include "kernels.hpp"

namespace {
typedef int a8i __attribute__((ext_vector_type(8)));
typedef float a4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ a8i load_operand(const uint8_t* blk, bool valid, int g) {
  a8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  if (valid) {
    const uint4 lo = *reinterpret_cast<const uint4*>(blk + 16 * g);
    const uint4 hi = *reinterpret_cast<const uint4*>(blk + 64 + 16 * g);
    r = a8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  return r;
}

// zero the 16-byte pieces of the operand outside bytes [lo, hi) of the block
__device__ __forceinline__ a8i keep_range(a8i v, int g, int lo, int hi) {
  const int b0 = 16 * g, b1 = 64 + 16 * g;
  if (!(b0 >= lo && b0 + 16 <= hi)) v[0] = v[1] = v[2] = v[3] = 0;
  if (!(b1 >= lo && b1 + 16 <= hi)) v[4] = v[5] = v[6] = v[7] = 0;
  return v;
}
}  // namespace

namespace fp8bs {

__global__ __launch_bounds__(256) void gemm_promotion_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    int64_t M, int64_t N, int64_t K, int64_t promote_k, float* __restrict__ C, int64_t ldc,
    int64_t tiles_n, int64_t tiles) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= tiles) return;
  const int64_t tm = wid / tiles_n, tn = wid % tiles_n;
  const int r = lane & 15, g = lane >> 4;
  const int64_t m = tm * 16 + r, n = tn * 16 + r;
  const bool vm = m < M, vn = n < N;
  const uint8_t* arow = A + (vm ? m : 0) * lda;
  const uint8_t* brow = B + (vn ? n : 0) * ldb;
  const int64_t KB = K / 128;
  const a4f zero = {0.f, 0.f, 0.f, 0.f};
  a4f acc = zero, chain = zero;
  if (promote_k >= 128) {
    const int64_t per = promote_k / 128;
    for (int64_t kb = 0; kb < KB; ++kb) {
      const a8i w = load_operand(brow + kb * 128, vn, g);
      const a8i x = load_operand(arow + kb * 128, vm, g);
      chain = mfma_e4m3_16x16x128(w, x, chain);
      if ((kb + 1) % per == 0 || kb + 1 == KB) {
        acc = acc + chain;
        chain = zero;
      }
    }
  } else {
    const int sub = (int)promote_k;
    for (int64_t kb = 0; kb < KB; ++kb) {
      const a8i w = load_operand(brow + kb * 128, vn, g);
      const a8i x = load_operand(arow + kb * 128, vm, g);
      for (int lo = 0; lo < 128; lo += sub) {
        const a4f P = mfma_e4m3_16x16x128(keep_range(w, g, lo, lo + sub), keep_range(x, g, lo, lo + sub), zero);
        acc = acc + P;
      }
    }
  }
  // lane holds outputs n = 16 tn + 4 g + v of row m = 16 tm + r
  const int64_t om = tm * 16 + r;
  if (om >= M) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t on = tn * 16 + 4 * g + v;
    if (on < N) C[om * ldc + on] = acc[v];
  }
}

hipError_t launch_gemm_promotion(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                                 int64_t M, int64_t N, int64_t K, int64_t promote_k, float* C,
                                 int64_t ldc, hipStream_t stream) {
  const int64_t tiles_n = (N + 15) / 16;
  const int64_t tiles = (M + 15) / 16 * tiles_n;
  const int64_t nblocks = (tiles + 3) / 4;
  hipLaunchKernelGGL(gemm_promotion_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream, A, lda,
                     B, ldb, M, N, K, promote_k, C, ldc, tiles_n, tiles);
  return hipGetLastError();
}

}  // namespace fp8bs
