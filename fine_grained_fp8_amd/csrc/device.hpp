// Device-side numerics shared by the quantizer and GEMM kernels (gfx950).
//
// Everything here is written for CDNA4 wave64: DPP row reductions over 16
// lanes, the hardware FP32 -> OCP E4M3 pack, and FP32 FMA.  Built with
// -ffp-contract=off so every rounding step is the one written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kCanonicalNaN = 0x7FC00000u;
constexpr uint32_t kScaleFloorBits = 0x2B8CBCCCu;   // fl32(1e-12)
constexpr uint32_t kBf16InfAbs = 0x7F80u;            // |x| bits above this are NaN

__device__ __forceinline__ float scale_floor() { return __uint_as_float(kScaleFloorBits); }

// Max over the 16 lanes of a DPP row (one 1x128 tile = 16 lanes x 8 BF16);
// every lane of the row ends with the row maximum.
// Per-half max of two packed u16 values over each group of 8 consecutive lanes
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, a),
                                                                __builtin_bit_cast(us2, b)));
}
__device__ __forceinline__ uint32_t row8_max_pk_u16(uint32_t t) {
  t = pk_max_u16(t, (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  t = pk_max_u16(t, (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  t = pk_max_u16(t, (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0x141, 0xF, 0xF, true));  // row_half_mirror
  return t;
}

__device__ __forceinline__ uint32_t row16_max_u32(uint32_t t) {
  t = max(t, (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  t = max(t, (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  t = max(t, (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0x141, 0xF, 0xF, true));  // row_half_mirror
  t = max(t, (uint32_t)__builtin_amdgcn_mov_dpp((int)t, 0x140, 0xF, 0xF, true));  // row_mirror
  return t;
}

// Max of |x| over the 8 BF16 values packed in four dwords, as BF16 magnitude
// bits (integer order of non-negative BF16 bit patterns is value order; NaN
// patterns sort above 0x7F80).
__device__ __forceinline__ uint32_t absmax_bits8(uint4 d) {
  us2 a = __builtin_bit_cast(us2, d.x & 0x7FFF7FFFu);
  us2 b = __builtin_bit_cast(us2, d.y & 0x7FFF7FFFu);
  us2 c = __builtin_bit_cast(us2, d.z & 0x7FFF7FFFu);
  us2 e = __builtin_bit_cast(us2, d.w & 0x7FFF7FFFu);
  us2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, e));
  uint32_t mm = __builtin_bit_cast(uint32_t, m);
  return max(mm & 0xFFFFu, mm >> 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// fl32(a / 448) for a finite non-negative BF16 value a: one Newton-Markstein
// correction of y = fl32(a * fl32(1/448)) (the remainder a - 448 y is exact
// with an FMA).  Equal to the IEEE quotient for every such a: checked
// exhaustively on the host (tests/c/check_div.c).  Three operations instead
// of a full correctly rounded division.
__device__ __forceinline__ float div448_bf16(float a) {
  constexpr float r448 = 1.0f / 448.0f;
  const float y = a * r448;
  const float e = __builtin_fmaf(-y, 448.0f, a);
  return __builtin_fmaf(e, r448, y);
}

// Online tile scale from the tile's |x| max bits: max(fl32(amax/448), floor);
// a NaN in the tile gives the canonical NaN (fmaxf would drop it), an
// infinite max the infinite scale.
__device__ __forceinline__ float tile_scale(uint32_t amax_bits) {
  if (amax_bits > kBf16InfAbs) return __uint_as_float(kCanonicalNaN);
  if (amax_bits == kBf16InfAbs) return __uint_as_float(0x7F800000u);
  return fmaxf(div448_bf16(__uint_as_float(amax_bits << 16)), scale_floor());
}

// fl32(1 / s) for a finite online scale s = tile_scale(amax): the hardware
// reciprocal estimate refined by one Newton step through FMAs.  Equal to the
// IEEE reciprocal for every scale the online rule can produce (all finite
// BF16 maxima and the floor): checked exhaustively on the GPU
// (fp8_probe_recip_online).
__device__ __forceinline__ float recip_online(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, r0, 1.0f);
  return __builtin_fmaf(e, r0, r0);
}

__device__ __forceinline__ float amax_value(uint32_t amax_bits) {
  return amax_bits > kBf16InfAbs ? __uint_as_float(kCanonicalNaN) : __uint_as_float(amax_bits << 16);
}

// fl32(x / s) for the online path, given r = fl32(1 / s).
// One Newton-Markstein correction of y = fl32(x * r): the remainder
// e = x - y * s is exact (FMA) and fl32(y + e * r) is the correctly rounded
// quotient.  Valid for s >= fl32(1e-12) from a BF16 amax and |x| <= amax;
// verified exhaustively on the host over that whole domain.  Only x = -0
// would lose its sign (-0 + +0 = +0), hence the copysign.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  float y = x * r;
  float e = __builtin_fmaf(-y, s, x);
  float q = __builtin_fmaf(e, r, y);
  return __builtin_copysignf(q, x);
}

// Saturating round-to-nearest-even FP32 -> E4M3 of two non-NaN values into
// byte pair `Hi` of `old`.  The explicit clamp makes finite overflow and
// +-Inf saturate to +-448 before the hardware pack.
template <bool Hi>
__device__ __forceinline__ int pack2_sat(float a, float b, int old) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, Hi);
}

// Four values -> one dword of codes (NaN-free inputs).
__device__ __forceinline__ uint32_t pack4_sat(float a, float b, float c, float d) {
  int w = pack2_sat<false>(a, b, 0);
  w = pack2_sat<true>(c, d, w);
  return (uint32_t)w;
}

// Four values -> one dword of codes, NaN inputs -> 0x7F.
__device__ __forceinline__ uint32_t pack4_sat_nan(float a, float b, float c, float d) {
  uint32_t w = pack4_sat(a, b, c, d);
  if (__builtin_isnan(a)) w = (w & 0xFFFFFF00u) | 0x7Fu;
  if (__builtin_isnan(b)) w = (w & 0xFFFF00FFu) | 0x7F00u;
  if (__builtin_isnan(c)) w = (w & 0xFF00FFFFu) | 0x7F0000u;
  if (__builtin_isnan(d)) w = (w & 0x00FFFFFFu) | 0x7F000000u;
  return w;
}

// One 16x16x128 FP8 MFMA, E4M3 x E4M3 with FP32 accumulation and no block
// scaling: D = A B + C.  The builtin names the block-scaled instruction;
// with both scale operands (and their op_sel) zero the compiler selects the
// plain v_mfma_f32_16x16x128_f8f6f4 instead, a single instruction where the
// scaled form issues a scale-load prefix as well (twice the issue cycles
// per MFMA).  The products are the same either way.
__device__ __forceinline__ v4f mfma_e4m3_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 4x4 byte transpose: rows a0..a3 (byte j of a_i = element (i, j)) ->
// columns o0..o3 (byte i of o_j = element (i, j)).
__device__ __forceinline__ void transpose4x4_bytes(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                                   uint32_t& o0, uint32_t& o1, uint32_t& o2, uint32_t& o3) {
  uint32_t t0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);   // a0c0 a1c0 a0c1 a1c1
  uint32_t t1 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);   // a2c0 a3c0 a2c1 a3c1
  uint32_t t2 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);   // a0c2 a1c2 a0c3 a1c3
  uint32_t t3 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);   // a2c2 a3c2 a2c3 a3c3
  o0 = __builtin_amdgcn_perm(t1, t0, 0x05040100u);
  o1 = __builtin_amdgcn_perm(t1, t0, 0x07060302u);
  o2 = __builtin_amdgcn_perm(t3, t2, 0x05040100u);
  o3 = __builtin_amdgcn_perm(t3, t2, 0x07060302u);
}

}  // namespace fp8bs
