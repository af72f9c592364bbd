// Matrix-unit rate probe: a loop of independent FP8 MFMAs with no memory
// traffic.  A measurement aid for the GEMM's roofline, not a step of the
// quantization method: it shows the rate the chip sustains for the GEMM's
// own instruction (v_mfma_scale_f32_16x16x128_f8f6f4) on given operand
// bytes, since the clock under load depends on the power the data draws.
#include "device.hpp"
#include "kernels.hpp"

namespace fp8bs {

namespace {
typedef int pv8i __attribute__((ext_vector_type(8)));
typedef float pv4f __attribute__((ext_vector_type(4)));
constexpr int kChains = 8;   // independent accumulators: the unit never waits on a result
}  // namespace

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, const uint8_t* __restrict__ codes,
                                                         float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const pv8i a = *reinterpret_cast<const pv8i*>(codes + 32 * lane);
  const pv8i b = *reinterpret_cast<const pv8i*>(codes + 2048 + 32 * lane);
  pv4f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = pv4f{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) sum += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

hipError_t launch_mfma_probe(int64_t workgroups, int iters, const uint8_t* codes, float* out,
                             hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, iters, codes, out);
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
