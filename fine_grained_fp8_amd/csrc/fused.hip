// Fprop with the 1x128 quantization of X fused into the GEMM: BF16 X in,
// BF16/FP32 Y out, the codes formed on chip (and optionally written out).
//
// Sources: "Online Quantization During Training" section 5 (whether online
// scaling is affordable depends on fusing it with the neighbouring kernels;
// fused and unfused forms are to be compared); "FP8 Mixed Precision:
// DeepSeek-V3 Training Architecture" section 3 (1x128 activation tiles,
// block products accumulated in FP32 with the two scales applied per K
// block).
//
// Design: one workgroup per 128 (m) x 128 (n) output tile, four waves of
// 64 x 64.  Per K block the workgroup loads its 128 rows of X as BF16 (each
// wave 32 rows, 16 lanes per 1x128 tile), quantizes them with the 1x128
// quantizer's arithmetic (same amax, scale, reciprocal and rounding, so the
// codes and scales are bit-identical to fp8_quant_act_1x128's) straight into
// an LDS stage, while the 128 weight rows of the block arrive in the same
// stage by DMA.  Two stages: block kb+1 is loaded and quantized while block
// kb is multiplied; one barrier per block.  The fold is the block GEMM's:
// acc = fma(P, sx[m] * sw, acc) with P one v_mfma_f32_16x16x128_f8f6f4.
// Every output tile's workgroup quantizes its X rows again (N/128 times in
// all); that repeated work is the price of fusion this kernel measures.
// Workgroups of column tile 0 can also write the codes and scales out.
#include "device.hpp"
#include "kernels.hpp"

namespace fp8bs {

namespace {
typedef __attribute__((address_space(3))) void* fq_lds_ptr_t;
typedef int fv4i __attribute__((ext_vector_type(4)));
constexpr uint32_t kFqRsrcWord3 = 0x00020000u;
constexpr int kFqTile = 128 * 128;            // codes of one 128 x 128 operand tile
constexpr int kFqXScale = 2 * kFqTile;        // 128 token scales
constexpr int kFqWScale = kFqXScale + 512;    // the weight block's scale (256 B DMA slot)
constexpr int kFqStage = kFqWScale + 256;

template <bool kOutF32>
__device__ __forceinline__ void fq_store4(void* C, int64_t ldc, int64_t m, int64_t n, int64_t N, const v4f& r) {
  if constexpr (kOutF32) {
    float* dst = reinterpret_cast<float*>(C) + m * ldc + n;
    if (n + 3 < N) {
      *reinterpret_cast<float4*>(dst) = make_float4(r[0], r[1], r[2], r[3]);
    } else {
      for (int v = 0; v < 4 && n + v < N; ++v) dst[v] = r[v];
    }
  } else {
    const __bf16 h[4] = {(__bf16)r[0], (__bf16)r[1], (__bf16)r[2], (__bf16)r[3]};
    uint16_t* dst = reinterpret_cast<uint16_t*>(C) + m * ldc + n;
    if (n + 3 < N) {
      const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, h[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, h[1]) << 16);
      const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, h[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, h[3]) << 16);
      *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
    } else {
      for (int v = 0; v < 4 && n + v < N; ++v) dst[v] = __builtin_bit_cast(uint16_t, h[v]);
    }
  }
}
}  // namespace

template <bool kOutF32>
__global__ __launch_bounds__(256, 1) void fused_quant_fprop_kernel(FusedFpropProblem p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2][kFqStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int nh = wave & 1, mh = wave >> 1;     // the wave's 64-column and 64-row halves
  const int64_t tiles_n = p.N / 128;
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * 128, n0 = (int64_t)(blockIdx.x % tiles_n) * 128;
  const int rows_m = (int)(p.M - m0 < 128 ? p.M - m0 : 128);
  const int KB = (int)(p.K / 128);

  // X: BF16, lane (sub, l16) = (lane >> 4, lane & 15) holds 8 values of row
  // 32 wave + 4 g + sub, columns 8 l16.., g = 0..7; rows past M read zero
  const __amdgpu_buffer_rsrc_t rsrc_x = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.X + m0 * p.ldx), (short)0, rows_m * (int)p.ldx * 2, (int)kFqRsrcWord3);
  const uint32_t off_x = (uint32_t)(((wave * 32 + (lane >> 4)) * (int)p.ldx + (lane & 15) * 8) * 2);
  // W: rows n0.. by DMA, 8 rows x 128 B per instruction, 16-byte chunks
  // XOR-swizzled by row & 7 (row & 7 == lane >> 3 here)
  const __amdgpu_buffer_rsrc_t rsrc_w = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.W + n0 * p.ldw), (short)0, 128 * (int)p.ldw, (int)kFqRsrcWord3);
  const uint32_t off_w = (uint32_t)((wave * 32 + (lane >> 3)) * (int)p.ldw + (((lane & 7) ^ (lane >> 3)) << 4));
  const __amdgpu_buffer_rsrc_t rsrc_sw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.sW + (n0 / 128) * p.ld_sw), (short)0, KB * 4, (int)kFqRsrcWord3);

  fv4i xq[8];
  auto load_block = [&](int kb, uint8_t* st) {
#pragma unroll
    for (int g = 0; g < 8; ++g)
      xq[g] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_x, off_x + (uint32_t)kb * 256u,
                                                    (uint32_t)g * 8u * (uint32_t)p.ldx, 0);
#pragma unroll
    for (int op = 0; op < 4; ++op)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_w, (fq_lds_ptr_t)(st + kFqTile + (wave * 4 + op) * 1024), 16,
                                               off_w + (uint32_t)kb * 128u, (uint32_t)(op * 8 * (int)p.ldw), 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_sw, (fq_lds_ptr_t)(st + kFqWScale), 4, (uint32_t)kb * 4u, 0, 0, 0);
  };
  // the 1x128 quantizer's arithmetic, tile by tile, into the stage
  auto quantize_block = [&](int kb, uint8_t* st) {
    const int sub = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint4 d = make_uint4((uint32_t)xq[g][0], (uint32_t)xq[g][1], (uint32_t)xq[g][2], (uint32_t)xq[g][3]);
      const uint32_t t = row16_max_u32(absmax_bits8(d));
      const float s = tile_scale(t);
      uint2 out;
      if (t < kBf16InfAbs) {
        const float r = recip_online(s);
        out.x = pack4_sat(div_by_scale(bf16_lo(d.x), s, r), div_by_scale(bf16_hi(d.x), s, r),
                          div_by_scale(bf16_lo(d.y), s, r), div_by_scale(bf16_hi(d.y), s, r));
        out.y = pack4_sat(div_by_scale(bf16_lo(d.z), s, r), div_by_scale(bf16_hi(d.z), s, r),
                          div_by_scale(bf16_lo(d.w), s, r), div_by_scale(bf16_hi(d.w), s, r));
      } else {
        out.x = pack4_sat_nan(bf16_lo(d.x) / s, bf16_hi(d.x) / s, bf16_lo(d.y) / s, bf16_hi(d.y) / s);
        out.y = pack4_sat_nan(bf16_lo(d.z) / s, bf16_hi(d.z) / s, bf16_lo(d.w) / s, bf16_hi(d.w) / s);
      }
      const int R = wave * 32 + 4 * g + sub;
      *reinterpret_cast<uint2*>(st + R * 128 + (((l16 >> 1) ^ (R & 7)) << 4) + (l16 & 1) * 8) = out;
      if (l16 == 0) reinterpret_cast<float*>(st + kFqXScale)[R] = s;
      if (p.q_out && n0 == 0 && R < rows_m) {
        *reinterpret_cast<uint2*>(p.q_out + (m0 + R) * p.ldq + kb * 128 + l16 * 8) = out;
        if (l16 == 0) p.s_out[kb * p.ld_s + m0 + R] = s;
      }
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int sw = lrow & 7;
  const int o_lo = ((lgrp ^ sw) << 4), o_hi = (((4 + lgrp) ^ sw) << 4);
  auto operand = [&](const uint8_t* tile, int row) {
    const fv4i lo = *reinterpret_cast<const fv4i*>(tile + row * 128 + o_lo);
    const fv4i hi = *reinterpret_cast<const fv4i*>(tile + row * 128 + o_hi);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  load_block(0, lds[0]);
  quantize_block(0, lds[0]);
  // the empty asm statements keep the compiler from moving LDS stores or
  // loads across the wait and the barrier (both builtins are memory-neutral
  // to it)
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  for (int kb = 0; kb < KB; ++kb) {
    uint8_t* cur = lds[kb & 1];
    uint8_t* nxt = lds[(kb + 1) & 1];
    const bool more = kb + 1 < KB;
    if (more) load_block(kb + 1, nxt);
    // block kb: the wave's 4 x 4 subtiles
    const float* sx = reinterpret_cast<const float*>(cur + kFqXScale);
    const float wsc = reinterpret_cast<const float*>(cur + kFqWScale)[0];
    v8i wop[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wop[i] = operand(cur + kFqTile, nh * 64 + i * 16 + lrow);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v8i xop = operand(cur, mh * 64 + j * 16 + lrow);
      const float c = sx[mh * 64 + j * 16 + lrow] * wsc;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        const v4f P = mfma_e4m3_16x16x128(wop[i], xop, zero);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(P[v], c, acc[i][j][v]);
      }
    }
    if (more) quantize_block(kb + 1, nxt);
    // block kb+1's codes written and its weights landed; every wave done
    // with block kb's stage before block kb+2 is loaded into it
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t m = m0 + mh * 64 + j * 16 + lrow;
    if (m >= p.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = n0 + nh * 64 + i * 16 + lgrp * 4;
      fq_store4<kOutF32>(p.C, p.ldc, m, n, p.N, acc[i][j]);
    }
  }
}

hipError_t launch_fused_quant_fprop(const FusedFpropProblem& p, hipStream_t stream) {
  const int64_t tiles = ((p.M + 127) / 128) * (p.N / 128);
  if (tiles == 0) return hipSuccess;
  if (p.out_fp32) {
    hipLaunchKernelGGL(fused_quant_fprop_kernel<true>, dim3((unsigned)tiles), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(fused_quant_fprop_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fp8bs
