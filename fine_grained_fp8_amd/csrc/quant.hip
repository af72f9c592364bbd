// Fine-grained FP8 quantizers for gfx950: 1x128 row tiles (online or with
// caller scales), 128x1 column tiles with transposed output, 128x128 weight
// blocks (optionally also writing the transposed codes), the amax-history
// update of the delayed-scaling policy, and the bare saturating E4M3 cast.
//
// Sources: "Fine-Grained FP8 Quantization in DeepSeek" sections 2-3 (1x128 tiles,
// 128x128 blocks, scale metadata produced efficiently and laid out for the
// GEMM); "FP8 Mixed Precision: DeepSeek-V3 Training Architecture" section 1
// (scale = block max / 448, clip to +-448); "Online Quantization During
// Training" sections 2 and 5 (max, scale and cast fused in one pass, right
// before the matmul).
#include "device.hpp"
#include "kernels.hpp"

namespace {
typedef int sv4i __attribute__((ext_vector_type(4)));
typedef int sv2i __attribute__((ext_vector_type(2)));
}  // namespace

namespace fp8bs {

// ---------------------------------------------------------------------------
// 1x128 row tiles.  One wave owns 4*kG rows x one 128-column K block: kG
// loads of 4 tiles each (a tile is one 16-lane DPP row holding 8 BF16 per
// lane), so the block's 4*kG scales are written as one contiguous store into
// the MN-major scale array [K/128][ld_s].  A workgroup's four waves take four
// consecutive K blocks of the same rows.
// ---------------------------------------------------------------------------
template <bool kExternal, int kG>
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t ldx, int64_t kblocks,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales, int64_t ld_s,
    const float* __restrict__ scales_in, float* __restrict__ amax_out,
    uint32_t* __restrict__ sat_count) {
  constexpr int kRows = 4 * kG;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nkbg = (kblocks + 3) >> 2;
  const int64_t rb = blockIdx.x / nkbg;
  const int64_t kb = (blockIdx.x % nkbg) * 4 + wave;
  if (kb >= kblocks) return;                 // whole wave idle; no block barriers below
  const int sub = lane >> 4;
  const int l16 = lane & 15;
  const int64_t r0 = rb * kRows;
  const uint16_t* xb = x + kb * 128 + l16 * 8;

  // The input is read once and the codes are written once: streaming
  // (non-temporal) accesses keep them from displacing cached data, which
  // measured ~6% faster with the input streamed from HBM.
  uint4 v[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const int64_t row = r0 + 4 * g + sub;
    const sv4i t = row < rows ? __builtin_nontemporal_load(reinterpret_cast<const sv4i*>(xb + row * ldx))
                              : sv4i{0, 0, 0, 0};
    v[g] = make_uint4((uint32_t)t[0], (uint32_t)t[1], (uint32_t)t[2], (uint32_t)t[3]);
  }

  float my_s = 0.0f, my_amax = 0.0f;
  uint32_t sat = 0;
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const int64_t row = r0 + 4 * g + sub;
    const uint32_t t = row16_max_u32(absmax_bits8(v[g]));
    float s;
    if constexpr (kExternal) {
      s = row < rows ? scales_in[kb * ld_s + row] : 1.0f;
    } else {
      s = tile_scale(t);
    }
    const uint4 d = v[g];
    uint2 out;
    if (!kExternal && t < kBf16InfAbs) {
      const float r = recip_online(s);       // correctly rounded reciprocal
      out.x = pack4_sat(div_by_scale(bf16_lo(d.x), s, r), div_by_scale(bf16_hi(d.x), s, r),
                        div_by_scale(bf16_lo(d.y), s, r), div_by_scale(bf16_hi(d.y), s, r));
      out.y = pack4_sat(div_by_scale(bf16_lo(d.z), s, r), div_by_scale(bf16_hi(d.z), s, r),
                        div_by_scale(bf16_lo(d.w), s, r), div_by_scale(bf16_hi(d.w), s, r));
    } else {
      // Inf/NaN tiles, or caller scales of any value: plain IEEE division.
      const float y0 = bf16_lo(d.x) / s, y1 = bf16_hi(d.x) / s;
      const float y2 = bf16_lo(d.y) / s, y3 = bf16_hi(d.y) / s;
      const float y4 = bf16_lo(d.z) / s, y5 = bf16_hi(d.z) / s;
      const float y6 = bf16_lo(d.w) / s, y7 = bf16_hi(d.w) / s;
      out.x = pack4_sat_nan(y0, y1, y2, y3);
      out.y = pack4_sat_nan(y4, y5, y6, y7);
      if constexpr (kExternal) {
        if (row < rows) {
          sat += (fabsf(y0) > 464.0f) + (fabsf(y1) > 464.0f) + (fabsf(y2) > 464.0f) +
                 (fabsf(y3) > 464.0f) + (fabsf(y4) > 464.0f) + (fabsf(y5) > 464.0f) +
                 (fabsf(y6) > 464.0f) + (fabsf(y7) > 464.0f);
        }
      }
    }
    if (row < rows)
      __builtin_nontemporal_store(sv2i{(int)out.x, (int)out.y},
                                  reinterpret_cast<sv2i*>(q + row * ldq + kb * 128 + l16 * 8));
    // lane j collects the scale of row r0 + j, held by lane 16 * (j % 4) in group j / 4
    const float sg = __shfl(s, (lane & 3) * 16);
    const float ag = __shfl(amax_value(t), (lane & 3) * 16);
    if ((lane >> 2) == g) { my_s = sg; my_amax = ag; }
  }
  const int64_t row = r0 + lane;
  if (lane < kRows && row < rows) {
    if (!kExternal) scales[kb * ld_s + row] = my_s;
    if (amax_out) amax_out[kb * ld_s + row] = my_amax;
  }
  if constexpr (kExternal) {
    if (sat_count) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sat += __shfl_xor(sat, off);
      if (lane == 0 && sat) atomicAdd(sat_count, sat);
    }
  }
}

// ---------------------------------------------------------------------------
// 128x1 column tiles, transposed output.  A workgroup stages a 128-row x
// 64-column BF16 block in LDS (coalesced 16-byte row loads).  Lane 8j + g of
// wave w then takes the column pair 8w + j over rows 16g..16g+15; the eight
// lanes of a pair combine the column max with DPP, and each writes 16 codes,
// so every store instruction covers whole 128-byte runs of eight transposed
// output rows.  LDS layout: 16-row group g starts at word 544*g (32 words of
// padding after every group) and its rows are rotated by 8*(g >> 1) words,
// which puts the 64 lanes of a column read on 64 distinct banks.
// ---------------------------------------------------------------------------
// Byte offset of the 16 transposed codes of column `col`, tokens
// 128 rb + 16 g .. + 15: row-major [cols][ldq], or operand-tiled (the
// transposed matrix has rows = columns of x and nbr 128-wide token blocks;
// these 16 codes fill one lane slot of its 2 KB tile).
template <bool kTiled>
__device__ __forceinline__ int64_t transposed_code_offset(int64_t col, int64_t rb, int g, int64_t ldq,
                                                          int64_t nbr) {
  if constexpr (kTiled)
    return ((col >> 4) * nbr + rb) * 2048 + (g >> 2) * 1024 + (((g & 3) << 4) + (col & 15)) * 16;
  else
    return col * ldq + rb * 128 + 16 * g;
}

// Operand-tiled store of a column pair's codes from lanes 8j + g (g = the
// 16-token group, o0 / o1 = columns col0 / col0 + 1): adjacent lanes g, g^1
// swap one value so that each store instruction covers 16 consecutive
// columns of one token group - whole 256-byte runs of the tiles - instead of
// every other 16-byte slot.
__device__ __forceinline__ uint4 swap_adjacent(uint4 v) {
  return make_uint4((uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, 0xB1, 0xF, 0xF, true),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, 0xB1, 0xF, 0xF, true),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.z, 0xB1, 0xF, 0xF, true),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.w, 0xB1, 0xF, 0xF, true));
}

template <bool kNontemporal>
__device__ __forceinline__ void store_pair_tiled(uint8_t* q, uint4 o0, uint4 o1, int64_t col0, int64_t rb,
                                                 int g, int64_t nbr) {
  const bool odd = g & 1;
  const uint4 recv = swap_adjacent(odd ? o0 : o1);
  const int64_t col = col0 + (odd ? 1 : 0);
  const uint4 a = odd ? recv : o0;           // token group g & ~1
  const uint4 b = odd ? o1 : recv;           // token group g | 1
  uint8_t* pa = q + transposed_code_offset<true>(col, rb, g & ~1, 0, nbr);
  uint8_t* pb = q + transposed_code_offset<true>(col, rb, g | 1, 0, nbr);
  if constexpr (kNontemporal) {
    __builtin_nontemporal_store(sv4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w}, reinterpret_cast<sv4i*>(pa));
    __builtin_nontemporal_store(sv4i{(int)b.x, (int)b.y, (int)b.z, (int)b.w}, reinterpret_cast<sv4i*>(pb));
  } else {
    *reinterpret_cast<uint4*>(pa) = a;
    *reinterpret_cast<uint4*>(pb) = b;
  }
}

__device__ __forceinline__ int cols_tile_word(int row, int word) {
  const int g = row >> 4;
  return g * 544 + (row & 15) * 32 + ((word + 8 * (g >> 1)) & 31);
}

template <bool kTiled>
__global__ __launch_bounds__(256) void quant_cols_kernel(
    const uint16_t* __restrict__ x, int64_t cols, int64_t ldx, int64_t ncb, int64_t nbr,
    int64_t nblocks, uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales,
    int64_t ld_s, float* __restrict__ amax_out) {
  __shared__ uint32_t tile[8 * 544];
  const int t = threadIdx.x;
  uint4 vals[4];
  auto load_block = [&](int64_t blk) {
    const int64_t lr0 = (blk / ncb) * 128, lc0 = (blk % ncb) * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = t + 256 * i;
      const int row = ci >> 3, cc = ci & 7;
      const int64_t col = lc0 + cc * 8;
      uint4 val = make_uint4(0, 0, 0, 0);
      const uint16_t* src = x + (lr0 + row) * ldx + col;
      if (col + 8 <= cols) {
        val = *reinterpret_cast<const uint4*>(src);
      } else if (col < cols) {               // ragged last chunk: stay inside the row
        uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int e = 0; e < 8 && col + e < cols; ++e) h[e] = src[e];
        val = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
      }
      vals[i] = val;
    }
  };
  // A workgroup takes blocks blockIdx.x, blockIdx.x + gridDim.x, ... (one
  // block each at the launch's grid; no registers held for a prefetch)
  for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
    load_block(blk);
    const int64_t rb = blk / ncb;
    const int64_t c0 = (blk % ncb) * 64;
    const int64_t r0 = rb * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = t + 256 * i;
      const int row = ci >> 3, cc = ci & 7;
      *reinterpret_cast<uint4*>(&tile[cols_tile_word(row, cc * 4)]) = vals[i];
    }
    __syncthreads();
    const int lane = t & 63, g = lane & 7;
    const int p = 8 * (t >> 6) + (lane >> 3);
    uint32_t d[16];
    us2 m = {0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      d[i] = tile[cols_tile_word(16 * g + i, p)];
      m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, d[i] & 0x7FFF7FFFu));
    }
    const uint32_t mm = row8_max_pk_u16(__builtin_bit_cast(uint32_t, m));
    uint4 outs[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t tt = h ? (mm >> 16) : (mm & 0xFFFFu);
      const float s = tile_scale(tt);
      float y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = h ? bf16_hi(d[i]) : bf16_lo(d[i]);
      uint4 out;
      if (tt < kBf16InfAbs) {
        const float r = recip_online(s);
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = div_by_scale(y[i], s, r);
        out.x = pack4_sat(y[0], y[1], y[2], y[3]);
        out.y = pack4_sat(y[4], y[5], y[6], y[7]);
        out.z = pack4_sat(y[8], y[9], y[10], y[11]);
        out.w = pack4_sat(y[12], y[13], y[14], y[15]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = y[i] / s;
        out.x = pack4_sat_nan(y[0], y[1], y[2], y[3]);
        out.y = pack4_sat_nan(y[4], y[5], y[6], y[7]);
        out.z = pack4_sat_nan(y[8], y[9], y[10], y[11]);
        out.w = pack4_sat_nan(y[12], y[13], y[14], y[15]);
      }
      outs[h] = out;
      const int64_t col = c0 + 2 * p + h;
      if (col < cols) {
        if constexpr (!kTiled) *reinterpret_cast<uint4*>(q + transposed_code_offset<false>(col, rb, g, ldq, nbr)) = out;
        if (g == 0) {
          scales[rb * ld_s + col] = s;
          if (amax_out) amax_out[rb * ld_s + col] = amax_value(tt);
        }
      }
    }
    // tiled output: cols % 128 == 0, so both columns exist
    if constexpr (kTiled) store_pair_tiled<false>(q, outs[0], outs[1], c0 + 2 * p, rb, g, nbr);
    __syncthreads();   // the next block overwrites the tile
  }
}

// ---------------------------------------------------------------------------
// Both orientations of the backward-pass activation from one read: for a
// 128x128 block, the 1x128 row tiles (Dgrad operand, row-major codes and
// MN-major scales) and the 128x1 column tiles (Wgrad operand, transposed
// codes).  The row tiles are quantized from registers exactly as in
// quant_rows_kernel (one 16-lane DPP row per tile row); the block is also
// staged in LDS, where eight lanes share two adjacent columns (16 rows each)
// and combine the column max with DPP.  Input and codes are streamed
// (non-temporal).  Every code and scale equals the one the separate row and
// column quantizers produce.  The 32 KB tile admits four workgroups per CU
// (measured: 31 KB would admit five), so the register bound is set for four:
// at five the operand-tiled form spilled a register into scratch.
// ---------------------------------------------------------------------------
template <bool kTiled>
__global__ __launch_bounds__(256, 4) void quant_dual_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t ncb, int64_t nbr, int64_t nblocks,
    uint8_t* __restrict__ q_row, int64_t ldq_row, float* __restrict__ s_row, int64_t ld_s_row,
    uint8_t* __restrict__ q_col, int64_t ldq_col, float* __restrict__ s_col, int64_t ld_s_col) {
  // BF16 pairs: word c of row r holds columns 2c, 2c+1 and sits at word
  // c ^ (8 * ((r >> 4) & 7)), so the column reads below hit 64 distinct banks
  __shared__ uint32_t tile[128][64];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int sub = lane >> 4, l16 = lane & 15;

  // ---- load: row wave*32 + 4i + sub, 8 BF16 at columns 8*l16.. ----
  uint4 v[8];
  auto load_block = [&](int64_t blk) {
    const int64_t r0 = (blk / ncb) * 128, c0 = (blk % ncb) * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = wave * 32 + 4 * i + sub;
      const sv4i u = __builtin_nontemporal_load(reinterpret_cast<const sv4i*>(x + (r0 + row) * ldx + c0 + l16 * 8));
      v[i] = make_uint4((uint32_t)u.x, (uint32_t)u.y, (uint32_t)u.z, (uint32_t)u.w);
    }
  };
  // A workgroup takes blocks blockIdx.x, blockIdx.x + gridDim.x, ... (one
  // block each at the launch's grid; no registers held for a prefetch)
  for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
    load_block(blk);
    const int64_t rb = blk / ncb;
    const int64_t kb = blk % ncb;
    const int64_t r0 = rb * 128, c0 = kb * 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = wave * 32 + 4 * i + sub;
      *reinterpret_cast<uint4*>(&tile[row][(l16 * 4) ^ (8 * ((row >> 4) & 7))]) = v[i];
    }

    // ---- 1x128 row tiles, from registers ----
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = wave * 32 + 4 * i + sub;
      const uint32_t ta = row16_max_u32(absmax_bits8(v[i]));
      const float s = tile_scale(ta);
      const uint4 d = v[i];
      uint2 out;
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
      __builtin_nontemporal_store(sv2i{(int)out.x, (int)out.y},
                                  reinterpret_cast<sv2i*>(q_row + (r0 + row) * ldq_row + c0 + l16 * 8));
      if (l16 == 0) s_row[kb * ld_s_row + r0 + row] = s;
    }
    __syncthreads();

    // ---- 128x1 column tiles, from LDS ----
    // Lane 8j + g of wave w takes column pair cp = 32*pass + 8w + j and rows
    // 16g..16g+15; the 8 lanes of a pair reduce its amax with DPP and then
    // write each column's 128 codes as one contiguous 128-byte run.
    const int g = lane & 7, j = lane >> 3;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int cp = 32 * pass + 8 * wave + j;
      uint32_t d[16];
      us2 m = {0, 0};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        d[i] = tile[16 * g + i][cp ^ (8 * g)];
        m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, d[i] & 0x7FFF7FFFu));
      }
      const uint32_t mm = row8_max_pk_u16(__builtin_bit_cast(uint32_t, m));
      uint4 outs[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t tt = h ? (mm >> 16) : (mm & 0xFFFFu);
        const float s = tile_scale(tt);
        uint32_t w[4];
        if (tt < kBf16InfAbs) {
          const float r = recip_online(s);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = div_by_scale(h ? bf16_hi(d[4 * k + e]) : bf16_lo(d[4 * k + e]), s, r);
            w[k] = pack4_sat(y[0], y[1], y[2], y[3]);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = (h ? bf16_hi(d[4 * k + e]) : bf16_lo(d[4 * k + e])) / s;
            w[k] = pack4_sat_nan(y[0], y[1], y[2], y[3]);
          }
        }
        const int64_t col = c0 + 2 * cp + h;
        outs[h] = make_uint4(w[0], w[1], w[2], w[3]);
        if constexpr (!kTiled)
          __builtin_nontemporal_store(sv4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]},
                                      reinterpret_cast<sv4i*>(q_col + transposed_code_offset<false>(col, rb, g, ldq_col, nbr)));
        if (g == 0) s_col[rb * ld_s_col + col] = s;
      }
      if constexpr (kTiled) store_pair_tiled<true>(q_col, outs[0], outs[1], c0 + 2 * cp, rb, g, nbr);
    }
    __syncthreads();   // the next block overwrites the tile
  }
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks: one workgroup per block, block max through DPP row
// reduction, cross-row shuffles and LDS; optional transposed codes via an LDS
// byte tile and 4x4 byte transposes (for the input-gradient GEMM).  kTiled
// writes both code matrices in the GEMM's operand-tiled layout instead of
// row-major: per 16 rows x 128 columns one 2 KB tile, whose 1 KB halves are
// what a wave's 64 lanes load as 16 bytes each (lane 16g + i: row i, columns
// 64h + 16g..).
// ---------------------------------------------------------------------------
template <bool kTiled>
__global__ __launch_bounds__(256) void quant_weight_kernel(
    const uint16_t* __restrict__ w, int64_t ldw, int64_t nbk, int64_t nbr,
    uint8_t* __restrict__ q, int64_t ldq, uint8_t* __restrict__ q_t, int64_t ldq_t,
    float* __restrict__ scales, int64_t ld_s) {
  __shared__ uint32_t wmax[4];
  __shared__ uint32_t codes[128][32];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int64_t bi = blockIdx.x / nbk, bj = blockIdx.x % nbk;
  const int64_t r0 = bi * 128, c0 = bj * 128;
  uint4 v[8];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ci = t + 256 * i;
    const int row = ci >> 4, cc = ci & 15;
    v[i] = *reinterpret_cast<const uint4*>(w + (r0 + row) * ldw + c0 + cc * 8);
    m = max(m, absmax_bits8(v[i]));
  }
  m = row16_max_u32(m);
  m = max(m, (uint32_t)__shfl_xor((int)m, 16));
  m = max(m, (uint32_t)__shfl_xor((int)m, 32));
  if (lane == 0) wmax[t >> 6] = m;
  __syncthreads();
  m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float s = tile_scale(m);
  if (t == 0) scales[bi * ld_s + bj] = s;
  const bool fast = m < kBf16InfAbs;
  const float r = fast ? recip_online(s) : 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ci = t + 256 * i;
    const int row = ci >> 4, cc = ci & 15;
    const uint4 d = v[i];
    uint2 out;
    if (fast) {
      out.x = pack4_sat(div_by_scale(bf16_lo(d.x), s, r), div_by_scale(bf16_hi(d.x), s, r),
                        div_by_scale(bf16_lo(d.y), s, r), div_by_scale(bf16_hi(d.y), s, r));
      out.y = pack4_sat(div_by_scale(bf16_lo(d.z), s, r), div_by_scale(bf16_hi(d.z), s, r),
                        div_by_scale(bf16_lo(d.w), s, r), div_by_scale(bf16_hi(d.w), s, r));
    } else {
      out.x = pack4_sat_nan(bf16_lo(d.x) / s, bf16_hi(d.x) / s, bf16_lo(d.y) / s, bf16_hi(d.y) / s);
      out.y = pack4_sat_nan(bf16_lo(d.z) / s, bf16_hi(d.z) / s, bf16_lo(d.w) / s, bf16_hi(d.w) / s);
    }
    if constexpr (kTiled) {
      // operand-tiled: 2 KB per 16 rows x 128 columns; this chunk (columns
      // 8cc..8cc+7 of the block) is half of lane slot (cc >> 1) & 3 of half cc >> 3
      const int64_t R = r0 + row;
      const int64_t off = ((R >> 4) * nbk + bj) * 2048 + (cc >> 3) * 1024 +
                          ((((cc >> 1) & 3) << 4) + (R & 15)) * 16 + (cc & 1) * 8;
      *reinterpret_cast<uint2*>(q + off) = out;
    } else {
      *reinterpret_cast<uint2*>(q + (r0 + row) * ldq + c0 + cc * 8) = out;
    }
    if (q_t) {
      codes[row][cc * 2] = out.x;
      codes[row][cc * 2 + 1] = out.y;
    }
  }
  if (!q_t) return;                          // uniform over the workgroup
  __syncthreads();
  const int cg = t & 31, rg = t >> 5;        // columns 4cg..4cg+3, rows 16rg..16rg+15
  uint32_t o[4][4];
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    const int rr = rg * 16 + qd * 4;
    transpose4x4_bytes(codes[rr][cg], codes[rr + 1][cg], codes[rr + 2][cg], codes[rr + 3][cg],
                       o[qd][0], o[qd][1], o[qd][2], o[qd][3]);
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const uint4 val = make_uint4(o[0][jj], o[1][jj], o[2][jj], o[3][jj]);
    if constexpr (kTiled) {
      // row R of the transposed matrix, its K block bi, 16 columns 16rg..: one lane slot
      const int64_t R = c0 + 4 * cg + jj;
      const int64_t off = ((R >> 4) * nbr + bi) * 2048 + (rg >> 2) * 1024 + (((rg & 3) << 4) + (R & 15)) * 16;
      *reinterpret_cast<uint4*>(q_t + off) = val;
    } else {
      *reinterpret_cast<uint4*>(q_t + (c0 + 4 * cg + jj) * ldq_t + r0 + 16 * rg) = val;
    }
  }
}

__global__ __launch_bounds__(256) void history_update_kernel(float* __restrict__ hist,
                                                             const float* __restrict__ amax,
                                                             int64_t n, float decay, int init,
                                                             float* __restrict__ scales_out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float h;
  if (init) {
    h = amax[i];
  } else {
    const float one_minus = 1.0f - decay;
    const float a = decay * hist[i];
    const float b = one_minus * amax[i];
    h = a + b;                                // separate roundings (no contraction)
  }
  hist[i] = h;
  if (scales_out) {
    float s = h / 448.0f;
    s = __builtin_isnan(s) ? __uint_as_float(kCanonicalNaN) : fmaxf(s, scale_floor());
    scales_out[i] = s;
  }
}

__global__ __launch_bounds__(256) void cast_e4m3_kernel(const float* __restrict__ x, int64_t n,
                                                        uint8_t* __restrict__ q) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    q[i] = (uint8_t)(pack4_sat_nan(x[i], 0.0f, 0.0f, 0.0f) & 0xFFu);
  }
}

// ----------------------------- launchers -----------------------------------

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                             const float* scales_in, float* amax_out, uint32_t* sat_count,
                             hipStream_t stream) {
  // 16 rows per wave: measured on 8192x7168 with the input streamed from HBM,
  // 16 rows run ~15% faster than 64 (more, shorter waves keep reads and
  // writes overlapped and leave a shorter tail)
  constexpr int kG = 4;
  const int64_t kblocks = cols / 128;
  const int64_t nblocks = ((rows + 4 * kG - 1) / (4 * kG)) * ((kblocks + 3) / 4);
  if (scales_in) {
    hipLaunchKernelGGL((quant_rows_kernel<true, kG>), dim3((unsigned)nblocks), dim3(256), 0, stream,
                       x, rows, ldx, kblocks, q, ldq, scales, ld_s, scales_in, amax_out, sat_count);
  } else {
    hipLaunchKernelGGL((quant_rows_kernel<false, kG>), dim3((unsigned)nblocks), dim3(256), 0, stream,
                       x, rows, ldx, kblocks, q, ldq, scales, ld_s, scales_in, amax_out, sat_count);
  }
  return hipGetLastError();
}

hipError_t launch_quant_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q_row, int64_t ldq_row, float* s_row, int64_t ld_s_row,
                             uint8_t* q_col, int64_t ldq_col, float* s_col, int64_t ld_s_col,
                             bool tiled, hipStream_t stream) {
  const int64_t ncb = cols / 128;
  const int64_t nblocks = (rows / 128) * ncb;
  const int64_t nbr = rows / 128;
  // one block per workgroup: two per workgroup (the second prefetched during
  // the first) measured 13% slower at X 4096x7168, whose 1792 blocks then
  // filled fewer than one round of the 4 resident workgroups per CU
  const int64_t grid = nblocks;
  if (tiled)
    hipLaunchKernelGGL(quant_dual_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, x, ldx, ncb,
                       nbr, nblocks, q_row, ldq_row, s_row, ld_s_row, q_col, ldq_col, s_col, ld_s_col);
  else
    hipLaunchKernelGGL(quant_dual_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, x, ldx, ncb,
                       nbr, nblocks, q_row, ldq_row, s_row, ld_s_row, q_col, ldq_col, s_col, ld_s_col);
  return hipGetLastError();
}

hipError_t launch_quant_cols(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                             float* amax_out, bool tiled, hipStream_t stream) {
  const int64_t ncb = (cols + 63) / 64;
  const int64_t nblocks = (rows / 128) * ncb;
  const int64_t nbr = rows / 128;
  const int64_t grid = nblocks;                // one block per workgroup (as the dual kernel)
  if (tiled)
    hipLaunchKernelGGL(quant_cols_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream,
                       x, cols, ldx, ncb, nbr, nblocks, q, ldq, scales, ld_s, amax_out);
  else
    hipLaunchKernelGGL(quant_cols_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream,
                       x, cols, ldx, ncb, nbr, nblocks, q, ldq, scales, ld_s, amax_out);
  return hipGetLastError();
}

hipError_t launch_quant_weight(const uint16_t* w, int64_t rows, int64_t cols, int64_t ldw,
                               uint8_t* q, int64_t ldq, uint8_t* q_t, int64_t ldq_t,
                               float* scales, int64_t ld_s, bool tiled, hipStream_t stream) {
  const int64_t nbk = cols / 128, nbr = rows / 128;
  const int64_t nblocks = nbr * nbk;
  if (tiled)
    hipLaunchKernelGGL(quant_weight_kernel<true>, dim3((unsigned)nblocks), dim3(256), 0, stream,
                       w, ldw, nbk, nbr, q, ldq, q_t, ldq_t, scales, ld_s);
  else
    hipLaunchKernelGGL(quant_weight_kernel<false>, dim3((unsigned)nblocks), dim3(256), 0, stream,
                       w, ldw, nbk, nbr, q, ldq, q_t, ldq_t, scales, ld_s);
  return hipGetLastError();
}

hipError_t launch_history_update(float* hist, const float* amax, int64_t n, float decay, int init,
                                 float* scales_out, hipStream_t stream) {
  const int64_t nblocks = (n + 255) / 256;
  hipLaunchKernelGGL(history_update_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream,
                     hist, amax, n, decay, init, scales_out);
  return hipGetLastError();
}

hipError_t launch_cast_e4m3(const float* x, int64_t n, uint8_t* q, hipStream_t stream) {
  int64_t nblocks = (n + 255) / 256;
  if (nblocks > 1048576) nblocks = 1048576;
  hipLaunchKernelGGL(cast_e4m3_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream, x, n, q);
  return hipGetLastError();
}

}  // namespace fp8bs
