// Activation quantization with a chosen tile size and percentile clipping.
//
// Sources: "Fine-Grained FP8 Quantization in DeepSeek", section 2 (one scale
// per tile of contiguous values) and its study lab (error against tile size,
// cost of the scale metadata); "Online Quantization During Training",
// section 4 (percentile clipping instead of the plain max).
//
// Tiles are 1 x T contiguous values of a row, T in {32, ..., 1024}.  The clip
// value c is the rank-th largest |x| of the tile (rank 1: the max, the online
// rule; the rank - 1 values above c saturate), s = max(fl32(c / 448),
// fl32(1e-12)), q = E4M3(fl32(x / s)).  A tile holding NaN gets scale NaN and
// NaN codes.  Scales are MN-major, [cols/T][ld_s], as for the 1x128 rule.
#include "device.hpp"
#include "kernels.hpp"

namespace {
typedef int tv4i __attribute__((ext_vector_type(4)));
typedef int tv2i __attribute__((ext_vector_type(2)));

// a >= b afterwards
__device__ __forceinline__ void cx(uint32_t& a, uint32_t& b) {
  const uint32_t hi = max(a, b), lo = min(a, b);
  a = hi;
  b = lo;
}

// Batcher's odd-even merge sort network for 8 keys, descending (19 exchanges)
__device__ __forceinline__ void sort8_desc(uint32_t k[8]) {
  cx(k[0], k[1]); cx(k[2], k[3]); cx(k[4], k[5]); cx(k[6], k[7]);
  cx(k[0], k[2]); cx(k[1], k[3]); cx(k[4], k[6]); cx(k[5], k[7]);
  cx(k[1], k[2]); cx(k[5], k[6]);
  cx(k[0], k[4]); cx(k[1], k[5]); cx(k[2], k[6]); cx(k[3], k[7]);
  cx(k[2], k[4]); cx(k[3], k[5]);
  cx(k[1], k[2]); cx(k[3], k[4]); cx(k[5], k[6]);
}

// k <- the 8 largest of k and p (both sorted descending), sorted descending:
// the pairwise max of k and reversed p is a bitonic sequence holding them,
// which three half-cleaner stages sort.
__device__ __forceinline__ void merge_top8(uint32_t k[8], const uint32_t p[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) k[i] = max(k[i], p[7 - i]);
#pragma unroll
  for (int d = 4; d > 0; d >>= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & d) == 0) cx(k[i], k[i + d]);
  }
}

__device__ __forceinline__ uint32_t key_lo(uint32_t w) { return w & 0x7FFFu; }
__device__ __forceinline__ uint32_t key_hi(uint32_t w) { return (w >> 16) & 0x7FFFu; }
}  // namespace

namespace fp8bs {

// A workgroup's four waves take four consecutive rows of one 1024-column
// chunk; lane l of a wave holds two runs of 8 consecutive BF16, at columns
// 8l and 512 + 8l of the chunk.  For T <= 512 each run belongs to its own
// group of T / 8 lanes (one tile); for T = 1024 both runs of all 64 lanes
// form the tile.
template <int T>
__global__ __launch_bounds__(256) void quant_tiles_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, int rank,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales, int64_t ld_s,
    uint32_t* __restrict__ sat_count, int64_t nchunks) {
  constexpr bool kJoint = T == 1024;
  constexpr int NT = kJoint ? 1 : 2;           // tiles a lane takes part in
  constexpr int L = kJoint ? 64 : T / 8;       // lanes per tile
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (blockIdx.x / nchunks) * 4 + wave;
  const int64_t chunk = blockIdx.x % nchunks;
  if (row >= rows) return;                     // whole wave
  const int64_t c0 = chunk * 1024 + lane * 8;
  bool valid[2];
  uint4 d[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    valid[h] = c0 + 512 * h < cols;            // tiles never straddle cols (cols % T == 0)
    d[h] = make_uint4(0, 0, 0, 0);
    if (valid[h]) {
      const tv4i u = __builtin_nontemporal_load(reinterpret_cast<const tv4i*>(x + row * ldx + c0 + 512 * h));
      d[h] = make_uint4((uint32_t)u.x, (uint32_t)u.y, (uint32_t)u.z, (uint32_t)u.w);
    }
  }

  uint32_t sat = 0;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    // the runs of this tile group: {j}, or both runs for T = 1024
    const int h0 = kJoint ? 0 : j, h1 = kJoint ? 1 : j;
    uint32_t lane_max = absmax_bits8(d[h0]);
    if (kJoint) lane_max = max(lane_max, absmax_bits8(d[h1]));

    uint32_t top0, ckey;
    if (rank == 1) {
      uint32_t m = lane_max;
#pragma unroll
      for (int off = 1; off < L; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
      top0 = ckey = m;
    } else {
      uint32_t k[8];
      {
        const uint4 a = d[h0];
        k[0] = key_lo(a.x); k[1] = key_hi(a.x); k[2] = key_lo(a.y); k[3] = key_hi(a.y);
        k[4] = key_lo(a.z); k[5] = key_hi(a.z); k[6] = key_lo(a.w); k[7] = key_hi(a.w);
        sort8_desc(k);
      }
      if (kJoint) {
        const uint4 a = d[h1];
        uint32_t p[8] = {key_lo(a.x), key_hi(a.x), key_lo(a.y), key_hi(a.y),
                         key_lo(a.z), key_hi(a.z), key_lo(a.w), key_hi(a.w)};
        sort8_desc(p);
        merge_top8(k, p);
      }
#pragma unroll
      for (int off = 1; off < L; off <<= 1) {
        uint32_t p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = (uint32_t)__shfl_xor((int)k[i], off);
        merge_top8(k, p);
      }
      top0 = k[0];
      ckey = k[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) ckey = (i == rank - 1) ? k[i] : ckey;
    }
    // a NaN anywhere in the tile gives the NaN scale whatever the rank
    const float s = tile_scale(top0 > kBf16InfAbs ? top0 : ckey);

#pragma unroll
    for (int h = h0; h <= h1; ++h) {
      const uint32_t w[4] = {d[h].x, d[h].y, d[h].z, d[h].w};
      float y[8];
      if (top0 < kBf16InfAbs) {
        const float r = recip_online(s);
        if (absmax_bits8(d[h]) <= ckey) {
          // every |x| <= c: the verified reciprocal shortcut
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[2 * e] = div_by_scale(bf16_lo(w[e]), s, r);
            y[2 * e + 1] = div_by_scale(bf16_hi(w[e]), s, r);
          }
        } else {
          // values above the clip value: plain IEEE division
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = bf16_lo(w[e]), b = bf16_hi(w[e]);
            y[2 * e] = key_lo(w[e]) <= ckey ? div_by_scale(a, s, r) : a / s;
            y[2 * e + 1] = key_hi(w[e]) <= ckey ? div_by_scale(b, s, r) : b / s;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[2 * e] = bf16_lo(w[e]) / s;
          y[2 * e + 1] = bf16_hi(w[e]) / s;
        }
      }
      uint2 out;
      if (top0 < kBf16InfAbs) {
        out.x = pack4_sat(y[0], y[1], y[2], y[3]);
        out.y = pack4_sat(y[4], y[5], y[6], y[7]);
      } else {
        out.x = pack4_sat_nan(y[0], y[1], y[2], y[3]);
        out.y = pack4_sat_nan(y[4], y[5], y[6], y[7]);
      }
      if (valid[h]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sat += fabsf(y[e]) > 464.0f;
        __builtin_nontemporal_store(tv2i{(int)out.x, (int)out.y},
                                    reinterpret_cast<tv2i*>(q + row * ldq + c0 + 512 * h));
      }
    }
    if (valid[h0] && (lane % L) == 0) scales[((c0 + 512 * h0) / T) * ld_s + row] = s;
  }
  if (sat_count) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sat += __shfl_xor(sat, off);
    if (lane == 0 && sat) atomicAdd(sat_count, sat);
  }
}

hipError_t launch_quant_tiles(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int tile,
                              int rank, uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                              uint32_t* sat_count, hipStream_t stream) {
  const int64_t nchunks = (cols + 1023) / 1024;
  const int64_t nblocks = (rows + 3) / 4 * nchunks;
  const dim3 grid((unsigned)nblocks), block(256);
  switch (tile) {
    case 32: hipLaunchKernelGGL(quant_tiles_kernel<32>, grid, block, 0, stream, x, rows, cols, ldx, rank, q, ldq, scales, ld_s, sat_count, nchunks); break;
    case 64: hipLaunchKernelGGL(quant_tiles_kernel<64>, grid, block, 0, stream, x, rows, cols, ldx, rank, q, ldq, scales, ld_s, sat_count, nchunks); break;
    case 128: hipLaunchKernelGGL(quant_tiles_kernel<128>, grid, block, 0, stream, x, rows, cols, ldx, rank, q, ldq, scales, ld_s, sat_count, nchunks); break;
    case 256: hipLaunchKernelGGL(quant_tiles_kernel<256>, grid, block, 0, stream, x, rows, cols, ldx, rank, q, ldq, scales, ld_s, sat_count, nchunks); break;
    case 512: hipLaunchKernelGGL(quant_tiles_kernel<512>, grid, block, 0, stream, x, rows, cols, ldx, rank, q, ldq, scales, ld_s, sat_count, nchunks); break;
    default: hipLaunchKernelGGL(quant_tiles_kernel<1024>, grid, block, 0, stream, x, rows, cols, ldx, rank, q, ldq, scales, ld_s, sat_count, nchunks); break;
  }
  return hipGetLastError();
}

}  // namespace fp8bs
