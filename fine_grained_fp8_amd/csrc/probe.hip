// Measurement and verification aids (declared in include/fp8bs_probe.h), not
// steps of the quantization method.
//
// mfma_probe_kernel: a loop of independent FP8 MFMAs with no memory traffic.
// It shows the rate the chip sustains for the GEMMs' instruction on given
// operand bytes (the clock under load depends on the power the data draws),
// and, by mode, what the instruction's encoding and the GEMMs' per-block
// FP32 fold cost in issue slots:
//   mode 0  plain v_mfma_f32_16x16x128_f8f6f4, 8 accumulator chains
//   mode 1  the block-scaled encoding of the same product (scales 2^0)
//   mode 2  plain MFMAs with a zero accumulator, each followed by the 4 FP32
//           FMAs that fold the partial of the same chain from the previous
//           round into its running sum (the GEMMs' instruction mix)
#include "device.hpp"
#include "kernels.hpp"

namespace fp8bs {

namespace {
constexpr int kChains = 8;   // independent accumulators: the unit never waits on a result
}  // namespace

template <int kMode>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, const uint8_t* __restrict__ codes,
                                                         float* __restrict__ out, float fold_scale) {
  const int lane = threadIdx.x & 63;
  const v8i a = *reinterpret_cast<const v8i*>(codes + 32 * lane);
  const v8i b = *reinterpret_cast<const v8i*>(codes + 2048 + 32 * lane);
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = zero;
  if constexpr (kMode == 2) {
    v4f Pa[kChains], Pb[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) Pa[c] = zero;
    // One round: a new partial per chain, each MFMA followed by the fold of
    // that chain's partial from the previous round (8 MFMAs old, complete).
    // Each chain's operand passes through an empty asm every round: with a
    // zero accumulator the products are otherwise identical and
    // loop-invariant, and the compiler would compute one of them once.
    v8i ar[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) ar[c] = a;
    auto round = [&](v4f (&Pn)[kChains], const v4f (&Pp)[kChains]) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) __asm__ volatile("" : "+v"(ar[c]));
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        Pn[c] = mfma_e4m3_16x16x128(ar[c], b, zero);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[c][v] = __builtin_fmaf(Pp[c][v], fold_scale, acc[c][v]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    int it = 0;
    for (; it + 1 < iters; it += 2) {
      round(Pb, Pa);
      round(Pa, Pb);
    }
    if (it < iters) {
      round(Pb, Pa);
#pragma unroll
      for (int c = 0; c < kChains; ++c) Pa[c] = Pb[c];
    }
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[c][v] = __builtin_fmaf(Pa[c][v], fold_scale, acc[c][v]);
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        if constexpr (kMode == 0) {
          acc[c] = mfma_e4m3_16x16x128(a, b, acc[c]);
        } else {
          // E8M0 127 = 2^0 on both operands: the scaled encoding, same product
          acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
        }
      }
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) sum += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

hipError_t launch_mfma_probe(int64_t workgroups, int iters, int mode, const uint8_t* codes, float* out,
                             hipStream_t stream) {
  const dim3 grid((unsigned)workgroups), block(256);
  switch (mode) {
    case 0: hipLaunchKernelGGL(mfma_probe_kernel<0>, grid, block, 0, stream, iters, codes, out, 1.0f); break;
    case 1: hipLaunchKernelGGL(mfma_probe_kernel<1>, grid, block, 0, stream, iters, codes, out, 1.0f); break;
    default: hipLaunchKernelGGL(mfma_probe_kernel<2>, grid, block, 0, stream, iters, codes, out, 1.0f); break;
  }
  return hipGetLastError();
}

// The quantizers' reciprocal of an online scale, element by element (for the
// exhaustive check that it equals the IEEE reciprocal on every such scale).
__global__ __launch_bounds__(256) void recip_online_probe_kernel(const float* __restrict__ s,
                                                                 float* __restrict__ r, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) r[i] = recip_online(s[i]);
}

hipError_t launch_recip_online_probe(const float* s, float* r, int64_t n, hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(recip_online_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, s, r, n);
  return hipGetLastError();
}

}  // namespace fp8bs
