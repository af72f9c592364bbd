// Block-scaled FP8 GEMM for gfx950 (FP8 MFMA, FP32 accumulation, per-128-K
// scale epilogue), in the Fprop, Dgrad and Wgrad layouts plus a grouped
// (per-expert) Fprop.
//
// Sources: "FP8 Mixed Precision: DeepSeek-V3 Training Architecture" section 3
// (E4M3 products, FP32 accumulators, block scale product applied to the
// accumulated sums); "Fine-Grained Quantization in DeepSeek" section 4
// (FP8 values and local scales loaded by the kernel, products accumulated in
// a wider type; scale application, transpose layout and epilogue decide the
// speed); "Introduction to LLM Quantization" section 2 steps 3-4 (block
// product on the matrix unit, then rescale by the block's factors) and
// section 1 (forward, input-gradient and weight-gradient products).
//
// Design (CDNA4):
//  * One v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, block scales 2^0)
//    covers exactly one 128-wide K block of a 16x16 output tile, so each
//    block's partial sum P comes out of a single MFMA with a zero accumulator
//    and is folded into the running FP32 total with one FMA per element:
//    acc = fma(P, sa * sb, acc) - the promotion to FP32 at every 128-element
//    interval that the method prescribes.  The MFMA's own E8M0 block scales
//    stay at 2^0 because the method's FP32 scales are not powers of two.
//  * The weight-side operand is the MFMA "A" (rows = output columns n) and the
//    token-side operand the MFMA "B" (columns = output rows m): each lane owns
//    4 consecutive n of one output row m (contiguous stores), and in
//    Fprop/Dgrad one weight-block scale per wave and K block.
//  * Workgroup tile 256 (n) x 256 (m) x 128 (k), eight wave64s.  Operand tiles
//    are staged in LDS in a 16-byte-chunk XOR swizzle (conflict-free for the
//    MFMA operand reads and for the transposing Dgrad stores) with two stages:
//    K block kb+1 streams into one stage while block kb is multiplied out of
//    the other; one barrier per K block.
//  * K-contiguous operands are loaded straight into LDS with
//    buffer_load_dwordx4 ... lds (no staging registers); the buffer range ends
//    at the last valid row, so ragged M/N tails read zeros.  Dgrad reads the
//    forward weight codes W_q [d_out][d_in] transposed: each thread loads
//    16 rows x 4 bytes, transposes 4x4 byte blocks with v_perm_b32 and writes
//    16-byte K-contiguous chunks.
//  * Workgroup ids are remapped so each XCD (ids congruent mod 8) walks a
//    contiguous, M-grouped run of tiles and its private L2 sees the reuse.
#include "device.hpp"
#include "kernels.hpp"

namespace fp8bs {

namespace {

constexpr int BM = 256;        // token rows per workgroup
constexpr int BN = 256;        // output columns per workgroup
constexpr int BK = 128;        // one scale block
constexpr int kThreads = 512;
constexpr int kTileBytes = 256 * BK;
constexpr int kStageBytes = 2 * kTileBytes + 2048;   // W tile, X tile, 2 x 256 scales
constexpr int kGroupM = 4;
constexpr uint32_t kRsrcWord3 = 0x00020000u;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t total) {
  // ids congruent mod 8 share an XCD; give each XCD a contiguous run of tiles
  if ((total & 7) != 0) return b;
  return (b & 7) * (total >> 3) + (b >> 3);
}

__device__ __forceinline__ void grouped_order(int64_t t, int64_t tiles_m, int64_t tiles_n,
                                              int64_t& tm, int64_t& tn) {
  const int64_t width = (int64_t)kGroupM * tiles_n;
  const int64_t grp = t / width;
  const int64_t first = grp * kGroupM;
  int64_t gsz = tiles_m - first;
  if (gsz > kGroupM) gsz = kGroupM;
  const int64_t r = t - grp * width;
  tm = first + r % gsz;
  tn = r / gsz;
}

__device__ __forceinline__ v8i read_operand(const uint8_t* tile, int row, int g) {
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + swz(row, 2 * g));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + swz(row, 2 * g + 1));
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Wave tile: WN output columns x WM output rows.  Wgrad uses 64 x 128 (fewer
// distinct per-column weight scales per lane), the others 128 x 64.
template <int kLayout>
struct WaveShape {
  static constexpr int WN = kLayout == kWgrad ? 64 : 128;
  static constexpr int WM = kLayout == kWgrad ? 128 : 64;
  static constexpr int NI = WN / 16;
  static constexpr int NJ = WM / 16;
  static constexpr int WAVES_N = BN / WN;
};

template <int kLayout, bool kOutF32, bool kGrouped>
__global__ __launch_bounds__(kThreads, 2) void block_gemm_kernel(GemmProblem p, int64_t total_tiles) {
  using S = WaveShape<kLayout>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave % S::WAVES_N, wm = wave / S::WAVES_N;
  const int64_t tiles_n = (p.N + BN - 1) / BN;

  // ---- tile coordinates ----
  const int64_t b = xcd_remap(blockIdx.x, gridDim.x);
  int64_t m0, m_end, n0;
  const uint8_t* Bp = p.B;
  const float* sBp = p.sB;
  if constexpr (kGrouped) {
    if (b >= total_tiles) return;
    int64_t cum = 0, lo = 0, hi = 0, ntm = 0;
    int g = 0;
    for (; g < p.groups; ++g) {
      lo = p.offsets[g];
      hi = p.offsets[g + 1];
      ntm = (hi - lo + BM - 1) / BM;
      if (b < cum + ntm * tiles_n) break;
      cum += ntm * tiles_n;
    }
    if (g >= p.groups) return;
    const int64_t local = b - cum;
    m0 = lo + (local / tiles_n) * BM;
    n0 = (local % tiles_n) * BN;
    m_end = hi;
    Bp += (int64_t)g * p.N * p.ldb;
    sBp += (int64_t)g * (p.N / 128) * (p.K / BK);
  } else {
    const int64_t tiles_m = (p.M + BM - 1) / BM;
    int64_t tm, tn;
    grouped_order(b, tiles_m, tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
    m_end = p.M;
  }
  const int KB = (int)(p.K / BK);
  const int rows_m = (int)(m_end - m0 < BM ? m_end - m0 : BM);   // valid token rows in the tile
  const int rows_n = (int)(p.N - n0 < BN ? p.N - n0 : BN);       // valid output columns

  // ---- operand streams (out-of-range rows read as zero) ----
  const __amdgpu_buffer_rsrc_t rsrc_x = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.A + m0 * p.lda), (short)0, rows_m * (int)p.lda, (int)kRsrcWord3);
  __amdgpu_buffer_rsrc_t rsrc_w;
  if constexpr (kLayout == kDgrad) {
    rsrc_w = __builtin_amdgcn_make_buffer_rsrc((void*)(Bp + n0), (short)0,
                                               (int)((p.K - 1) * p.ldb) + rows_n, (int)kRsrcWord3);
  } else {
    rsrc_w = __builtin_amdgcn_make_buffer_rsrc((void*)(Bp + n0 * p.ldb), (short)0,
                                               rows_n * (int)p.ldb, (int)kRsrcWord3);
  }
  // this lane's slot in each of the wave's 4 load instructions (8 rows x 128 B each)
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);      // wave-uniform (SGPR)
  const int lrow8 = wave * 32 + (lane >> 3);
  const int lslot = lane & 7;
  const int cq = tid & 63, kg = tid >> 6;      // Dgrad: columns 4cq.., k rows 16kg..
  uint32_t rwt[16];

  auto issue_loads = [&](int kb, int stage) {
    uint8_t* st = smem + stage * kStageBytes;
    const int soff = kb * BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = lrow8 + j * 8;
      const int lc = lslot ^ ((row ^ (row >> 3)) & 7);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_x, (lds_ptr_t)(st + kTileBytes + (wave_u * 32 + j * 8) * 128),
                                               16, (uint32_t)(row * (int)p.lda + lc * 16), soff, 0, 0);
    }
    if constexpr (kLayout == kDgrad) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        rwt[i] = __builtin_amdgcn_raw_buffer_load_b32(
            rsrc_w, (uint32_t)((kb * BK + kg * 16 + i) * (int)p.ldb + cq * 4), 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = lrow8 + j * 8;
        const int lc = lslot ^ ((row ^ (row >> 3)) & 7);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_w, (lds_ptr_t)(st + (wave_u * 32 + j * 8) * 128),
                                                 16, (uint32_t)(row * (int)p.ldb + lc * 16), soff, 0, 0);
      }
    }
    // token-side scales of this K block, rows m0..m0+255 (contiguous in the MN-major layout)
    if (wave_u == 0) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.sA + (int64_t)kb * p.ld_sa + m0), (short)0, rows_m * 4, (int)kRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(st + 2 * kTileBytes), 16,
                                               (uint32_t)(lane * 16), 0, 0, 0);
    }
    if constexpr (kLayout == kWgrad) {
      if (wave_u == 1) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(sBp + (int64_t)kb * p.ld_sb + n0), (short)0, rows_n * 4, (int)kRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(st + 2 * kTileBytes + 1024), 16,
                                                 (uint32_t)(lane * 16), 0, 0, 0);
      }
    }
  };
  auto store_dgrad_w = [&](int stage) {
    uint8_t* st = smem + stage * kStageBytes;
    uint32_t o[4][4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
      transpose4x4_bytes(rwt[4 * qd], rwt[4 * qd + 1], rwt[4 * qd + 2], rwt[4 * qd + 3],
                         o[qd][0], o[qd][1], o[qd][2], o[qd][3]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4*>(st + swz(cq * 4 + j, kg)) = make_uint4(o[0][j], o[1][j], o[2][j], o[3][j]);
  };

  // weight-block scale (Fprop / Dgrad): one value per wave and K block
  const int nblk_last = (int)(p.N / 128) - 1;
  int wblk = (int)((n0 + wn * S::WN) / 128);
  wblk = wblk < nblk_last ? wblk : nblk_last;
  auto weight_scale = [&](int kb) -> float {
    if constexpr (kLayout == kFprop) return sBp[(int64_t)wblk * p.ld_sb + kb];
    else if constexpr (kLayout == kDgrad) return sBp[(int64_t)kb * p.ld_sb + wblk];
    else return 0.f;
  };

  const int lrow = lane & 15, lgrp = lane >> 4;
  v4f acc[S::NI][S::NJ];
#pragma unroll
  for (int i = 0; i < S::NI; ++i)
#pragma unroll
    for (int j = 0; j < S::NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  float wsc = weight_scale(0);
  issue_loads(0, 0);
  if constexpr (kLayout == kDgrad) store_dgrad_w(0);

  for (int kb = 0; kb < KB; ++kb) {
    const int stage = kb & 1;
    __builtin_amdgcn_s_waitcnt(0);           // this wave's loads for block kb have landed
    __syncthreads();                         // ... and every other wave's; stage kb^1 is free
    const bool more = kb + 1 < KB;
    float wsc_next = 0.f;
    if (more) {
      wsc_next = weight_scale(kb + 1);
      issue_loads(kb + 1, stage ^ 1);
    }
    const uint8_t* wt = smem + stage * kStageBytes;
    const uint8_t* xt = wt + kTileBytes;
    const float* sxl = reinterpret_cast<const float*>(wt + 2 * kTileBytes);
    const float* swl = sxl + 256;

    v8i bx[S::NJ];
    float c[S::NJ];
#pragma unroll
    for (int j = 0; j < S::NJ; ++j) {
      const int r = wm * S::WM + j * 16 + lrow;
      bx[j] = read_operand(xt, r, lgrp);
      c[j] = kLayout == kWgrad ? sxl[r] : sxl[r] * wsc;
    }
#pragma unroll
    for (int i = 0; i < S::NI; ++i) {
      const v8i a = read_operand(wt, wn * S::WN + i * 16 + lrow, lgrp);
      float4 rs = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (kLayout == kWgrad)
        rs = *reinterpret_cast<const float4*>(swl + wn * S::WN + i * 16 + lgrp * 4);
#pragma unroll
      for (int j = 0; j < S::NJ; ++j) {
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        const v4f P = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bx[j], zero, 0, 0,
                                                                      0, 127, 0, 127);
        if constexpr (kLayout == kWgrad) {
          acc[i][j][0] = __builtin_fmaf(P[0] * rs.x, c[j], acc[i][j][0]);
          acc[i][j][1] = __builtin_fmaf(P[1] * rs.y, c[j], acc[i][j][1]);
          acc[i][j][2] = __builtin_fmaf(P[2] * rs.z, c[j], acc[i][j][2]);
          acc[i][j][3] = __builtin_fmaf(P[3] * rs.w, c[j], acc[i][j][3]);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(P[v], c[j], acc[i][j][v]);
        }
      }
    }
    if (more) {
      if constexpr (kLayout == kDgrad) store_dgrad_w(stage ^ 1);
      wsc = wsc_next;
    }
  }

  // ---- epilogue: round and store ----
#pragma unroll
  for (int j = 0; j < S::NJ; ++j) {
    const int64_t m = m0 + wm * S::WM + j * 16 + lrow;
    if (m >= m_end) continue;
#pragma unroll
    for (int i = 0; i < S::NI; ++i) {
      const int64_t n = n0 + wn * S::WN + i * 16 + lgrp * 4;
      if (n >= p.N) continue;
      const v4f r = acc[i][j];
      if constexpr (kOutF32) {
        float* dst = reinterpret_cast<float*>(p.C) + m * p.ldc + n;
        if (n + 3 < p.N) {
          *reinterpret_cast<float4*>(dst) = make_float4(r[0], r[1], r[2], r[3]);
        } else {
          for (int v = 0; v < 4 && n + v < p.N; ++v) dst[v] = r[v];
        }
      } else {
        __bf16 h0 = (__bf16)r[0], h1 = (__bf16)r[1], h2 = (__bf16)r[2], h3 = (__bf16)r[3];
        const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
        const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, h2) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
        uint16_t* dst = reinterpret_cast<uint16_t*>(p.C) + m * p.ldc + n;
        if (n + 3 < p.N) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
        } else {
          const uint16_t hv[4] = {(uint16_t)(w0 & 0xFFFF), (uint16_t)(w0 >> 16),
                                  (uint16_t)(w1 & 0xFFFF), (uint16_t)(w1 >> 16)};
          for (int v = 0; v < 4 && n + v < p.N; ++v) dst[v] = hv[v];
        }
      }
    }
  }
}

template <int kLayout, bool kGrouped>
hipError_t launch_typed(const GemmProblem& p, hipStream_t stream, int64_t grid, int64_t total) {
  if (p.out_fp32) {
    hipLaunchKernelGGL((block_gemm_kernel<kLayout, true, kGrouped>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, p, total);
  } else {
    hipLaunchKernelGGL((block_gemm_kernel<kLayout, false, kGrouped>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, p, total);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream) {
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  if (p.groups > 0) {
    // upper bound on per-group M tiles without reading the device offsets
    const int64_t total = ((p.M + BM - 1) / BM + p.groups) * tiles_n;
    const int64_t grid = (total + 7) / 8 * 8;
    return launch_typed<kFprop, true>(p, stream, grid, total);
  }
  const int64_t tiles_m = (p.M + BM - 1) / BM;
  const int64_t total = tiles_m * tiles_n;
  switch (p.layout) {
    case kFprop: return launch_typed<kFprop, false>(p, stream, total, total);
    case kDgrad: return launch_typed<kDgrad, false>(p, stream, total, total);
    default: return launch_typed<kWgrad, false>(p, stream, total, total);
  }
}

}  // namespace fp8bs
