// FP8 token payloads: per-token messages [E4M3 codes | FP32 tile scales] for
// activations kept for the backward pass and for the MoE dispatch, their
// unpacking into the GEMM operand layout, and their restoration to BF16.
//
// Sources: "FP8 Mixed Precision: DeepSeek-V3 Training Architecture" section 4
// (activations cached in FP8; tokens quantized to FP8 on the fly before the
// expert all-to-all) and its section on the MoE all-to-all (a dispatched token
// is one hidden vector); "Fine-Grained FP8 Quantization in DeepSeek" section 2
// (the 1x128 tile scale travels with its codes).
//
// Message of a token with H channels: bytes [0, H) are the codes of its
// 1x128 tiles (the rule of the row quantizer), bytes [H, H + 4 H/128) the
// tiles' FP32 scales, little-endian, in tile order.
#include "device.hpp"
#include "kernels.hpp"

namespace {
typedef int pv4i __attribute__((ext_vector_type(4)));
typedef int pv2i __attribute__((ext_vector_type(2)));
constexpr int kChunk = 16;   // tiles per workgroup column chunk in the unpacker
// tiles per wave in the packer: 4 keeps enough workgroups in flight (8192
// messages of 7168 channels: 16 -> 8 -> 4 tiles measured 51 -> 43 -> 40 us)
constexpr int kPackChunk = 4;
}  // namespace

namespace fp8bs {

// ---------------------------------------------------------------------------
// Pack.  Lane group sub (16 lanes) of a wave owns one message; the wave walks
// kPackChunk consecutive tiles of it (one 16-lane DPP row per tile, 8 BF16 per
// lane, the arithmetic of quant_rows_kernel), keeps tile i's scale in lane i
// and writes the chunk's scales as one contiguous run.  A workgroup's four
// waves take four consecutive chunks of the same four messages.
// Message t carries source row src_rows[t] (or t); a source row outside
// [0, x_rows) gives NaN codes and NaN scales.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_tokens_kernel(
    const uint16_t* __restrict__ x, int64_t x_rows, int64_t ldx, int64_t kblocks,
    const int32_t* __restrict__ src_rows, int64_t T, uint8_t* __restrict__ msg, int64_t stride,
    int64_t nchunk_groups) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane >> 4, l16 = lane & 15;
  const int64_t t = (blockIdx.x / nchunk_groups) * 4 + sub;
  const int64_t kb0 = ((blockIdx.x % nchunk_groups) * 4 + wave) * kPackChunk;
  if (kb0 >= kblocks || t >= T) return;
  const int64_t src = src_rows ? (int64_t)src_rows[t] : t;
  const bool bad = src < 0 || src >= x_rows;
  const int64_t H = kblocks * 128;
  uint8_t* m = msg + t * stride;
  const uint16_t* xr = x + (bad ? 0 : src) * ldx + l16 * 8;

  uint4 v[kPackChunk];
#pragma unroll
  for (int i = 0; i < kPackChunk; ++i) {
    v[i] = make_uint4(0, 0, 0, 0);
    if (!bad && kb0 + i < kblocks) {
      const pv4i u = __builtin_nontemporal_load(reinterpret_cast<const pv4i*>(xr + (kb0 + i) * 128));
      v[i] = make_uint4((uint32_t)u.x, (uint32_t)u.y, (uint32_t)u.z, (uint32_t)u.w);
    }
  }
  float my_scale = __uint_as_float(0x7FC00000u);
#pragma unroll
  for (int i = 0; i < kPackChunk; ++i) {
    if (kb0 + i >= kblocks) break;
    uint2 out;
    float s;
    if (bad) {
      out = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
      s = __uint_as_float(0x7FC00000u);
    } else {
      const uint32_t ta = row16_max_u32(absmax_bits8(v[i]));
      s = tile_scale(ta);
      const uint4 d = v[i];
      if (ta < kBf16InfAbs) {
        const float r = recip_online(s);
        out.x = pack4_sat(div_by_scale(bf16_lo(d.x), s, r), div_by_scale(bf16_hi(d.x), s, r),
                          div_by_scale(bf16_lo(d.y), s, r), div_by_scale(bf16_hi(d.y), s, r));
        out.y = pack4_sat(div_by_scale(bf16_lo(d.z), s, r), div_by_scale(bf16_hi(d.z), s, r),
                          div_by_scale(bf16_lo(d.w), s, r), div_by_scale(bf16_hi(d.w), s, r));
      } else {
        out.x = pack4_sat_nan(bf16_lo(d.x) / s, bf16_hi(d.x) / s, bf16_lo(d.y) / s, bf16_hi(d.y) / s);
        out.y = pack4_sat_nan(bf16_lo(d.z) / s, bf16_hi(d.z) / s, bf16_lo(d.w) / s, bf16_hi(d.w) / s);
      }
    }
    __builtin_nontemporal_store(pv2i{(int)out.x, (int)out.y},
                                reinterpret_cast<pv2i*>(m + (kb0 + i) * 128 + l16 * 8));
    if (l16 == i) my_scale = s;
  }
  if (l16 < kPackChunk && kb0 + l16 < kblocks) *reinterpret_cast<float*>(m + H + 4 * (kb0 + l16)) = my_scale;
}

// ---------------------------------------------------------------------------
// Unpack into the GEMM operand layout: codes [T][ldq] and MN-major scales
// [H/128][ld_s].  A workgroup moves 16 messages x 16 tiles: 8 x 16-byte code
// pieces per thread, and one scale per thread (thread 16j + u takes tile j
// of message u, so each tile's 16 scales are one contiguous 64-byte run).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void unpack_tokens_kernel(
    const uint8_t* __restrict__ msg, int64_t T, int64_t kblocks, int64_t stride,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales, int64_t ld_s,
    int64_t nchunks) {
  const int tid = threadIdx.x;
  const int64_t t0 = (blockIdx.x / nchunks) * 16;
  const int64_t kb0 = (blockIdx.x % nchunks) * kChunk;
  const int64_t H = kblocks * 128;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int piece = tid + 256 * i;            // 16 messages x 128 pieces of 16 bytes
    const int64_t t = t0 + (piece >> 7);
    const int64_t off = kb0 * 128 + (int64_t)(piece & 127) * 16;
    if (t < T && off < H) {
      const pv4i u = *reinterpret_cast<const pv4i*>(msg + t * stride + off);
      *reinterpret_cast<pv4i*>(q + t * ldq + off) = u;
    }
  }
  const int64_t t = t0 + (tid & 15);
  const int64_t kb = kb0 + (tid >> 4);
  if (t < T && kb < kblocks)
    scales[kb * ld_s + t] = *reinterpret_cast<const float*>(msg + t * stride + H + 4 * kb);
}

// ---------------------------------------------------------------------------
// Restore BF16: y = RNE_bf16(decode(q) * s), rounded once from the exact
// product.  When s >= 2**-117 (exponent field >= 10) the product p = fl32(q s)
// and its residual fma(q, s, -p) are exact (no underflow), and the residual
// decides the one case FP32 rounding hides: p landing exactly on a BF16
// midpoint.  Smaller scales take an integer path: the E4M3 significand
// (<= 4 bits) times the FP32 significand (24 bits) fits 28 bits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t bf16_of_product_fast(float v, float s) {
  const float p = v * s;
  const float e = __builtin_fmaf(v, s, -p);
  const uint32_t b = __float_as_uint(p);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  if ((b & 0xFFFFu) == 0x8000u && e != 0.0f) {
    const bool above = (e > 0.0f) == (p > 0.0f);   // magnitude past the midpoint
    return (above ? b + 0x8000u : b) >> 16;
  }
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __noinline__ uint32_t bf16_of_product_small(uint32_t code, uint32_t sbits) {
  if ((code & 0x7Fu) == 0x7Fu) return 0x7FC0u;
  const uint32_t sign = ((code >> 7) ^ (sbits >> 31)) & 1u;
  const uint32_t e4 = (code >> 3) & 15u, m3 = code & 7u;
  const uint64_t mv = e4 ? 8u + m3 : m3;
  const int ev = e4 ? (int)e4 - 10 : -9;
  const uint32_t es = (sbits >> 23) & 0xFFu;
  const uint64_t ms = es ? ((sbits & 0x7FFFFFu) | 0x800000u) : (sbits & 0x7FFFFFu);
  const int e = ev + (es ? (int)es - 150 : -149);       // value = mv * ms * 2**e
  const uint64_t m = mv * ms;
  if (m == 0) return sign << 15;
  const int lead = 63 - __builtin_clzll(m);
  const int vexp = lead + e;
  const int lsb = (vexp > -126 ? vexp : -126) - 7;       // BF16 spacing exponent
  const int shift = lsb - e;                              // <= 25
  uint64_t k;
  if (shift <= 0) {
    k = m << (-shift);
  } else {
    k = m >> shift;
    const uint64_t rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (k & 1))) ++k;
  }
  const float r = __builtin_ldexpf((float)k, lsb);       // k <= 256: exact
  return (__float_as_uint(r) >> 16) | (sign << 15);
}

// Lane l of a wave restores codes [16 l, 16 l + 16) of a 1024-code chunk;
// a workgroup's four waves take four consecutive chunks of one message.
__global__ __launch_bounds__(256) void dequant_tokens_kernel(
    const uint8_t* __restrict__ msg, int64_t T, int64_t H, int64_t stride,
    uint16_t* __restrict__ y, int64_t ldy, int64_t ngroups) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = blockIdx.x / ngroups;
  const int64_t c = ((blockIdx.x % ngroups) * 4 + wave) * 1024 + lane * 16;
  if (t >= T || c >= H) return;
  const uint8_t* m = msg + t * stride;
  const pv4i u = *reinterpret_cast<const pv4i*>(m + c);
  const float s = *reinterpret_cast<const float*>(m + H + 4 * (c >> 7));
  const uint32_t sbits = __float_as_uint(s);
  const uint32_t w[4] = {(uint32_t)u.x, (uint32_t)u.y, (uint32_t)u.z, (uint32_t)u.w};
  uint32_t o[8];
  if (((sbits >> 23) & 0xFFu) >= 10u) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);   // bytes 0, 1
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);    // bytes 2, 3
      o[2 * k] = bf16_of_product_fast(lo[0], s) | (bf16_of_product_fast(lo[1], s) << 16);
      o[2 * k + 1] = bf16_of_product_fast(hi[0], s) | (bf16_of_product_fast(hi[1], s) << 16);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) b[e] = bf16_of_product_small((w[k] >> (8 * e)) & 0xFFu, sbits);
      o[2 * k] = b[0] | (b[1] << 16);
      o[2 * k + 1] = b[2] | (b[3] << 16);
    }
  }
  pv4i* dst = reinterpret_cast<pv4i*>(y + t * ldy + c);
  dst[0] = pv4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
  dst[1] = pv4i{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
}

hipError_t launch_pack_tokens(const uint16_t* x, int64_t x_rows, int64_t H, int64_t ldx,
                              const int32_t* src_rows, int64_t T, uint8_t* msg, int64_t stride,
                              hipStream_t stream) {
  const int64_t kblocks = H / 128;
  const int64_t nchunks = (kblocks + kPackChunk - 1) / kPackChunk;
  const int64_t ngroups = (nchunks + 3) / 4;
  const int64_t nblocks = (T + 3) / 4 * ngroups;
  hipLaunchKernelGGL(pack_tokens_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream, x, x_rows,
                     ldx, kblocks, src_rows, T, msg, stride, ngroups);
  return hipGetLastError();
}

hipError_t launch_unpack_tokens(const uint8_t* msg, int64_t T, int64_t H, int64_t stride,
                                uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                                hipStream_t stream) {
  const int64_t kblocks = H / 128;
  const int64_t nchunks = (kblocks + kChunk - 1) / kChunk;
  const int64_t nblocks = (T + 15) / 16 * nchunks;
  hipLaunchKernelGGL(unpack_tokens_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream, msg, T,
                     kblocks, stride, q, ldq, scales, ld_s, nchunks);
  return hipGetLastError();
}

hipError_t launch_dequant_tokens(const uint8_t* msg, int64_t T, int64_t H, int64_t stride,
                                 uint16_t* y, int64_t ldy, hipStream_t stream) {
  const int64_t ngroups = (H + 4095) / 4096;
  const int64_t nblocks = T * ngroups;
  hipLaunchKernelGGL(dequant_tokens_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream, msg, T,
                     H, stride, y, ldy, ngroups);
  return hipGetLastError();
}

}  // namespace fp8bs
