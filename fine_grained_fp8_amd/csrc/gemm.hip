// Block-scaled FP8 GEMM for gfx950 (FP8 MFMA, FP32 accumulation, per-128-K
// scale epilogue), in the Fprop, Dgrad and Wgrad layouts plus a grouped
// (per-expert) Fprop.
//
// Sources: "FP8 Mixed Precision: DeepSeek-V3 Training Architecture" section 3
// (E4M3 products, FP32 accumulators, block scale product applied to the
// accumulated sums); "Fine-Grained FP8 Quantization in DeepSeek" section 4
// (FP8 values and local scales loaded by the kernel, products accumulated in
// a wider type; scale application, transpose layout and epilogue decide the
// speed); "Introduction to LLM Quantization" section 2 steps 3-4 (block
// product on the matrix unit, then rescale by the block's factors) and
// section 1 (forward, input-gradient and weight-gradient products).
//
// Design (CDNA4):
//  * One v_mfma_f32_16x16x128_f8f6f4 (E4M3 x E4M3, no block scaling) covers
//    exactly one 128-wide K block of a 16x16 output tile, so each block's
//    partial sum P comes out of a single MFMA with a zero accumulator and is
//    folded into the running FP32 total with one FMA per element:
//    acc = fma(P, sa * sb, acc) - the promotion to FP32 at every 128-element
//    interval that the method prescribes.  The instruction's block-scaled
//    form is not used: the method's FP32 scales are not powers of two, and
//    its scale-load prefix would double the issue cost of every MFMA.
//  * The weight-side operand is the MFMA "A" (rows = output columns n) and the
//    token-side operand the MFMA "B" (columns = output rows m): each lane owns
//    4 consecutive n of one output row m, and in Fprop/Dgrad one weight-block
//    scale per wave and K block.
//  * Workgroup tile 256 (n) x 128 (m) x 128 (k): four wave64s, one per SIMD,
//    with the full 512-register budget each.
//  * block_gemm_direct_kernel (Fprop, Dgrad from W_q^T, Wgrad, grouped): each
//    wave's 64 weight-side rows go straight from memory into registers, the
//    shared token-side tile through four LDS stages by DMA; persistent over
//    tiles; details at the kernel.
//  * block_gemm_kernel (Dgrad reading W_q as stored): both tiles through
//    three LDS stages by DMA (buffer_load_dwordx4 ... lds, no staging
//    registers), each stage its own LDS object so the compiler sees that the
//    DMA into one stage never aliases reads of another; waves 128 x 64; the
//    weight tile is DMA'd as stored ([k][n]) and ds_read_b64_tr_b8 transposes
//    it on the way into the MFMA operand registers.
//  * Buffer ranges end at the last valid row, so ragged M/N tails read zeros.
//    LDS tiles store 16-byte chunks XOR-swizzled by row & 7 (conflict-free
//    operand reads).  The scales of each K block (contiguous in the MN-major
//    layout) ride along in the same stage.
//  * Tile ids are remapped so each XCD (ids congruent mod 8) walks a
//    contiguous, M-grouped run of tiles and its private L2 sees the reuse.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace fp8bs {

namespace {

constexpr int BM = 128;        // token rows per workgroup
constexpr int BN = 256;        // output columns per workgroup
constexpr int BK = 128;        // one scale block
constexpr int kThreads = 256;
constexpr int kWTile = BN * BK;   // 32 KB
constexpr int kXTile = BM * BK;   // 16 KB
constexpr int kScaleBytes = 2048; // token scales [256] + weight-side scales [256]
constexpr int kGroupM = 8;   // a power of two
static_assert((kGroupM & (kGroupM - 1)) == 0, "GroupM order masks with kGroupM - 1");
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// Wave tile: 128 output columns (n) x 64 output rows (m); waves 2 (n) x 2 (m).
constexpr int WN = 128, WM = 64, NI = WN / 16, NJ = WM / 16;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t total) {
  // ids congruent mod 8 share an XCD; give each XCD a contiguous run of tiles
  if ((total & 7) != 0) return b;
  return (b & 7) * (total >> 3) + (b >> 3);
}

// GroupM order: tile t of a tiles_m x tiles_n grid walks groups of kGroupM
// M tiles, column by column.  32-bit arithmetic (the host keeps tile counts
// below 2^31): each 64-bit division by a runtime value is a long software
// sequence, and this runs at every tile boundary.
__device__ __forceinline__ void grouped_order(int64_t t64, int64_t tiles_m64, int64_t tiles_n64,
                                              int64_t& tm, int64_t& tn) {
  const uint32_t t = (uint32_t)t64, tiles_m = (uint32_t)tiles_m64, tiles_n = (uint32_t)tiles_n64;
  const uint32_t width = (uint32_t)kGroupM * tiles_n;
  const uint32_t grp = t / width;
  const uint32_t first = grp * (uint32_t)kGroupM;
  const uint32_t r = t - grp * width;
  const uint32_t gsz = tiles_m - first < (uint32_t)kGroupM ? tiles_m - first : (uint32_t)kGroupM;
  if (gsz == (uint32_t)kGroupM) {   // every group but a ragged last one
    tm = first + (r & (kGroupM - 1));
    tn = r / (uint32_t)kGroupM;
  } else {
    tm = first + r % gsz;
    tn = r / gsz;
  }
}

__device__ __forceinline__ v8i join(const v4i& lo, const v4i& hi) {
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ v4i lo_half(const v8i& v) { return v4i{v[0], v[1], v[2], v[3]}; }
__device__ __forceinline__ v4i hi_half(const v8i& v) { return v4i{v[4], v[5], v[6], v[7]}; }
__device__ __forceinline__ v8i pair(const uint8_t* lo_p, const uint8_t* hi_p) {
  const v4i lo = *reinterpret_cast<const v4i*>(lo_p);
  const v4i hi = *reinterpret_cast<const v4i*>(hi_p);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Dgrad weight tile kept as stored, [128 k][256 n] bytes, 16-byte chunks of a
// row XOR-swizzled by k & 7.  ds_read_b64_tr_b8 turns it into MFMA "A"
// operands: within each 16-lane group, lane r names row M[r] (8 bytes) and
// output lane j receives byte b of M[2b + (j >> 3)][j & 7].  Pointing even
// lanes at (k0 + r/2, n..n+7) and odd lanes at (k0 + r/2, n+8..n+15) gives
// lane j the 8 consecutive k of column n + j - the same k order as the
// K-contiguous operands.
__device__ __forceinline__ v8i read_operand_t(const uint8_t* tile, int n_sub, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int c16 = n_sub >> 4;
  v8i out;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int k = g * 32 + t * 8 + (j >> 1);
    const uint8_t* src = tile + k * 256 + ((c16 ^ (k & 7)) << 4) + 8 * (j & 1);
    const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(src));
    out[2 * t] = r[0];
    out[2 * t + 1] = r[1];
  }
  return out;
}

// Output tile `b` (0 <= b < the tile count): token rows [m0, min(m0 + BM,
// m_end)) and output columns [n0, n0 + BN); Bp / sBp point at the tile's
// group in the grouped case.  Tiles are numbered group by group (grouped) or
// in the GroupM-swizzled order.  Returns false when b lies past the last
// group.
__device__ __forceinline__ bool decode_tile_index(const GemmProblem& p, bool grouped, int64_t b,
                                                  int64_t& m0, int64_t& m_end, int64_t& n0,
                                                  const uint8_t*& Bp, const float*& sBp) {
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  Bp = p.B;
  sBp = p.sB;
  if (grouped) {
    // Offsets come from device memory unchecked: clamp each group into
    // [0, M] with hi >= lo, so a malformed array can only empty or overlap
    // groups, never move a row access outside A, sA or C.
    int64_t cum = 0, lo = 0, hi = 0, ntm = 0;
    int g = 0;
    for (; g < p.groups; ++g) {
      lo = min(max((int64_t)p.offsets[g], (int64_t)0), p.M);
      hi = min(max((int64_t)p.offsets[g + 1], lo), p.M);
      ntm = (hi - lo + BM - 1) / BM;
      if (b < cum + ntm * tiles_n) break;
      cum += ntm * tiles_n;
    }
    if (g >= p.groups) return false;
    // within a group, the GroupM order of the plain layouts: a round of an
    // XCD's workgroups covers 8 M tiles x fewer N tiles, so less of the
    // expert's weights per round
    int64_t tm, tn;
    grouped_order(b - cum, ntm, tiles_n, tm, tn);
    m0 = lo + tm * BM;
    n0 = tn * BN;
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
  return true;
}

// Grouped launches with at most kLdsGroups groups keep each group's clamped
// row range and first tile index in LDS, built once per workgroup; the tile
// decode then finds a tile's group with one compare per lane and a ballot
// instead of a loop of dependent reads of the offsets in global memory.
constexpr int kLdsGroups = 64;
struct GroupLds {
  int32_t* cum;   // [groups + 1]: tiles before group g
  int32_t* lo;    // [groups]: clamped first row
  int32_t* hi;    // [groups]: clamped end row
};

// Fill the table (wave 0; the caller's barrier publishes it).  Same clamping
// as decode_tile_index.
__device__ __forceinline__ void build_group_lds(const GemmProblem& p, const GroupLds& t, int lane) {
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  int32_t cnt = 0;
  if (lane < p.groups) {
    const int64_t lo = min(max((int64_t)p.offsets[lane], (int64_t)0), p.M);
    const int64_t hi = min(max((int64_t)p.offsets[lane + 1], lo), p.M);
    t.lo[lane] = (int32_t)lo;
    t.hi[lane] = (int32_t)hi;
    cnt = (int32_t)((hi - lo + BM - 1) / BM * tiles_n);
  }
  int32_t incl = cnt;   // inclusive scan over the wave's lanes
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane < p.groups) t.cum[lane + 1] = incl;
  if (lane == 0) t.cum[0] = 0;
}

// decode_tile_index for a grouped launch through the LDS table.
__device__ __forceinline__ bool decode_tile_lds(const GemmProblem& p, const GroupLds& t, int lane, int64_t b,
                                                int64_t& m0, int64_t& m_end, int64_t& n0,
                                                const uint8_t*& Bp, const float*& sBp) {
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  bool hit = false;
  if (lane < p.groups) hit = t.cum[lane] <= b && b < t.cum[lane + 1];   // empty groups never hit
  const uint64_t mask = __ballot(hit);
  if (mask == 0) return false;
  const int g = __builtin_amdgcn_readfirstlane(__builtin_ctzll(mask));
  const int64_t lo = t.lo[g], hi = t.hi[g];
  int64_t tm, tn;
  grouped_order(b - t.cum[g], (hi - lo + BM - 1) / BM, tiles_n, tm, tn);
  m0 = lo + tm * BM;
  n0 = tn * BN;
  m_end = hi;
  Bp = p.B + (int64_t)g * p.N * p.ldb;
  sBp = p.sB + (int64_t)g * (p.N / 128) * (p.K / BK);
  return true;
}

// Number of output tiles of a grouped launch, from the offsets as clamped by
// decode_tile_index.
__device__ __forceinline__ int64_t grouped_tile_count(const GemmProblem& p) {
  const int64_t tiles_n = (p.N + BN - 1) / BN;
  int64_t cum = 0;
  for (int g = 0; g < p.groups; ++g) {
    const int64_t lo = min(max((int64_t)p.offsets[g], (int64_t)0), p.M);
    const int64_t hi = min(max((int64_t)p.offsets[g + 1], lo), p.M);
    cum += (hi - lo + BM - 1) / BM * tiles_n;
  }
  return cum;
}

// Tile of workgroup id `id` in a one-tile-per-workgroup launch of `ids`
// workgroups; false for the padding ids of a grouped launch.
__device__ __forceinline__ bool decode_tile(const GemmProblem& p, int64_t total_tiles, bool grouped,
                                            int64_t id, int64_t ids,
                                            int64_t& m0, int64_t& m_end, int64_t& n0,
                                            const uint8_t*& Bp, const float*& sBp) {
  const int64_t b = xcd_remap(id, ids);
  if (grouped && b >= total_tiles) return false;
  return decode_tile_index(p, grouped, b, m0, m_end, n0, Bp, sBp);
}

// Round and store 4 consecutive outputs (n..n+3) of row m; columns past N
// are dropped.
// Values every lane holds alike, pinned to scalar registers (the tile
// decode runs 64-bit divisions on the vector unit).
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* v) {
  return reinterpret_cast<T*>(uniform_i64(reinterpret_cast<int64_t>(v)));
}

template <bool kOutF32>
__device__ __forceinline__ void store4(const GemmProblem& p, int64_t m, int64_t n, const v4f& r) {
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

// s_waitcnt immediate (gfx9 encoding): wait until at most `vm` vector-memory
// operations of this wave are outstanding and all LDS/scalar ones are done.
template <int vm>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(vm >= 0 && vm < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((vm & 15) | (7 << 4) | (0 << 8) | ((vm >> 4) << 14));
}

// the same with no wait on the LDS / scalar-memory counter
template <int vm>
__device__ __forceinline__ void wait_vm() {
  static_assert(vm >= 0 && vm < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((vm & 15) | (7 << 4) | (15 << 8) | ((vm >> 4) << 14));
}

template <int kLayout, bool kOutF32, bool kGrouped>
__global__ __launch_bounds__(kThreads, 1) void block_gemm_kernel(GemmProblem p, int64_t total_tiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_w0[kWTile];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_w1[kWTile];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_w2[kWTile];
  // X-tile objects carry the stage's scale vectors after the codes (fewer
  // distinct DMA targets for the compiler's wait tracking)
  __shared__ __attribute__((aligned(1024))) uint8_t lds_x0[kXTile + kScaleBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_x1[kXTile + kScaleBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_x2[kXTile + kScaleBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;

  // ---- tile coordinates ----
  int64_t m0, m_end, n0;
  const uint8_t* Bp;
  const float* sBp;
  if (!decode_tile(p, total_tiles, kGrouped, blockIdx.x, gridDim.x, m0, m_end, n0, Bp, sBp)) return;
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
  // Per-lane byte offsets of the wave's DMA instructions (1 KB each: 8 rows of
  // a K-contiguous tile, or 4 k-rows of the Dgrad tile).  With the row & 7
  // swizzle a lane's chunk is the same in every instruction, so instructions
  // differ by a uniform row stride.  The whole offset goes into the per-lane
  // VGPR offset, which is what the buffer range check applies to.
  const int xrow = wave * 32 + (lane >> 3);                          // + 8 j, j < 4
  const uint32_t off_x = (uint32_t)(xrow * (int)p.lda + (((lane & 7) ^ (lane >> 3)) << 4));
  uint32_t off_w, off_w_odd = 0;
  if constexpr (kLayout == kDgrad) {
    const int k = wave * 32 + (lane >> 4);                           // + 4 j, j < 8
    off_w = (uint32_t)(k * (int)p.ldb + (((lane & 15) ^ (k & 7)) << 4));
    off_w_odd = (uint32_t)(k * (int)p.ldb + (((lane & 15) ^ ((k + 4) & 7)) << 4));
  } else {
    const int wrow = wave * 64 + (lane >> 3);                        // + 8 j, j < 8
    off_w = (uint32_t)(wrow * (int)p.ldb + (((lane & 7) ^ (lane >> 3)) << 4));
  }
  const int w_kstride = kLayout == kDgrad ? BK * (int)p.ldb : BK;   // bytes per K block
  const int w_jstride = kLayout == kDgrad ? 4 * (int)p.ldb : 8 * (int)p.ldb;

  // weight-block scales (Fprop / Dgrad), read through a range-checked buffer
  const int64_t nb0 = n0 / 128;
  // Lanes 0 and 1 fetch the scales of n-blocks nb0 and nb0 + 1 (every other
  // lane repeats block nb0 + 2).  A block past the last one lies past the end
  // of the buffer, so the range check returns zero for it - no branch needed.
  const uint32_t sw_lane = (uint32_t)(nb0 + (lane < 2 ? lane : 2));
  const uint32_t sw_off = kLayout == kFprop ? sw_lane * (uint32_t)p.ld_sb * 4u : sw_lane * 4u;
  const uint32_t sw_kstride = kLayout == kFprop ? 4u : (uint32_t)p.ld_sb * 4u;
  const int64_t sw_elems = kLayout == kFprop ? (p.N / 128) * p.ld_sb : (p.K / BK) * p.ld_sb;
  const __amdgpu_buffer_rsrc_t rsrc_sw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)sBp, (short)0, kLayout == kWgrad ? 0 : (int)(sw_elems * 4), (int)kRsrcWord3);

  // Every wave issues the same number of DMA instructions per K block (the
  // scale vectors are loaded by all four waves; they write identical bytes),
  // so one vmcnt threshold fits every wave.  issue_load(kb, op, ...) issues
  // DMA instruction `op` of block kb: 0-3 token rows, 4-11 weight rows, 12
  // the token-side scales, 13 the weight-side scales.
  constexpr int kOpsPerBlock = 4 + 8 + 1 + 1;
  auto issue_load = [&](int kb, int op, uint8_t* wst, uint8_t* xst) {
    float* sst = reinterpret_cast<float*>(xst + kXTile);
    if (op < 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_x, (lds_ptr_t)(xst + (wave * 4 + op) * 1024), 16,
                                               off_x + (uint32_t)(kb * BK + op * 8 * (int)p.lda), 0, 0, 0);
    } else if (op < 12) {
      const int j = op - 4;
      const uint32_t ow = (kLayout == kDgrad && (j & 1)) ? off_w_odd : off_w;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_w, (lds_ptr_t)(wst + (wave * 8 + j) * 1024), 16,
                                               ow + (uint32_t)(kb * w_kstride + j * w_jstride), 0, 0, 0);
    } else if (op == 12) {
      // token-side scales of this K block, rows m0..m0+127 (contiguous in the MN-major layout)
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.sA + (int64_t)kb * p.ld_sa + m0), (short)0, rows_m * 4, (int)kRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(sst), 16, (uint32_t)(lane * 16), 0, 0, 0);
    } else if constexpr (kLayout == kWgrad) {
      // per-column weight-side scales of this K block, columns n0..n0+255
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(sBp + (int64_t)kb * p.ld_sb + n0), (short)0, rows_n * 4, (int)kRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(sst + 256), 16, (uint32_t)(lane * 16), 0, 0, 0);
    } else {
      // the two weight-block scales of this K block (n-blocks n0/128 and
      // n0/128 + 1) land in sst[256..257]
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_sw, (lds_ptr_t)(sst + 256), 4,
                                               sw_off + (uint32_t)kb * sw_kstride, 0, 0, 0);
    }
  };
  auto issue_loads = [&](int kb, uint8_t* wst, uint8_t* xst) {
#pragma unroll
    for (int op = 0; op < kOpsPerBlock; ++op) issue_load(kb, op, wst, xst);
  };

  const int lrow = lane & 15, lgrp = lane >> 4;
  // swizzled LDS addresses of this lane's operand rows: row & 7 == lrow & 7 for
  // every subtile, so subtile j (i) sits a constant 2048 B further on
  const int sw = lrow & 7;
  const int x_lo = (wm * WM + lrow) * 128 + (((2 * lgrp) ^ sw) << 4);
  const int x_hi = (wm * WM + lrow) * 128 + (((2 * lgrp + 1) ^ sw) << 4);
  const int w_lo = (wn * WN + lrow) * 128 + (((2 * lgrp) ^ sw) << 4);
  const int w_hi = (wn * WN + lrow) * 128 + (((2 * lgrp + 1) ^ sw) << 4);

  v4f acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // ---- one K block out of stage (wt, xt, sxl); block kb+2 streams into (wnx, xnx, snx) ----
  auto step = [&](int kb, const uint8_t* wt, const uint8_t* xt, uint8_t* wnx, uint8_t* xnx) {
    const float* sxl = reinterpret_cast<const float*>(xt + kXTile);
    wait_vm_lgkm0<kOpsPerBlock>();   // block kb landed; the next block may still fly
    const bool live = kb < KB;        // false for the padding steps
    // Bare barrier: __syncthreads() would add a release fence, i.e. a full
    // vmcnt(0) drain of the DMA still in flight for later blocks.  The waits
    // above already make this wave's block-kb data visible; the empty asm
    // keeps the compiler from moving LDS accesses across the barrier.
    // sched_barrier(0): nothing (MFMAs and folds included) is moved across
    // the step boundary by the instruction scheduler
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // All LDS reads of this block first, then the DMA for block kb+2: no LDS
    // read follows a DMA issue inside a step, so the compiler never has to
    // guess whether they alias (it would drain the DMA with vmcnt(0)).
    const float* swl = sxl + 256;
    float wsc = 0.f;
    if constexpr (kLayout != kWgrad) wsc = swl[(int)((n0 + wn * WN) / 128 - nb0)];
    v8i bx[NJ];
    float c[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      bx[j] = pair(xt + x_lo + j * 2048, xt + x_hi + j * 2048);
      const float t = sxl[wm * WM + j * 16 + lrow];
      c[j] = live ? (kLayout == kWgrad ? t : t * wsc) : 0.f;
    }
    v8i a[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (kLayout == kDgrad) a[i] = read_operand_t(wt, wn * WN + i * 16, lane);
      else a[i] = pair(wt + w_lo + i * 2048, wt + w_hi + i * 2048);
    }
    float4 rs[NI];
    if constexpr (kLayout == kWgrad) {
#pragma unroll
      for (int i = 0; i < NI; ++i) rs[i] = *reinterpret_cast<const float4*>(swl + wn * WN + i * 16 + lgrp * 4);
    }
    __asm__ volatile("" ::: "memory");
    // Block kb+2 streams into the stage freed by block kb-1.  The last two
    // steps have no block kb+2; they reload block KB-1 into that free stage
    // (in bounds, never read) so the DMA stays unconditional and keeps its
    // place between the MFMAs.
    const int kb_pf = kb + 2 < KB ? kb + 2 : KB - 1;

    // Software pipeline over the 8 subtile rows: the MFMAs of row i, each
    // followed by the FP32 fold of row i-1's partial sum in the same column
    // (issued four MFMAs earlier, so already complete), with two of block
    // kb+2's DMA instructions per row.  The matrix core, the VALU and the
    // vector-memory unit then work side by side instead of in turns.
    auto fold = [&](int i, int j, const v4f& P) {
      if constexpr (kLayout == kWgrad) {
        acc[i][j][0] = __builtin_fmaf(P[0] * rs[i].x, c[j], acc[i][j][0]);
        acc[i][j][1] = __builtin_fmaf(P[1] * rs[i].y, c[j], acc[i][j][1]);
        acc[i][j][2] = __builtin_fmaf(P[2] * rs[i].z, c[j], acc[i][j][2]);
        acc[i][j][3] = __builtin_fmaf(P[3] * rs[i].w, c[j], acc[i][j][3]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(P[v], c[j], acc[i][j][v]);
      }
    };
    v4f P0[NJ], P1[NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      v4f (&Pc)[NJ] = (i & 1) ? P1 : P0;
      v4f (&Pp)[NJ] = (i & 1) ? P0 : P1;
      // operands in AGPRs (the MFMA reads them there), leaving the VGPRs to
      // the accumulators and the partial sums the VALU folds
      __asm__ volatile("" : "+a"(a[i]));
      if (i == 0) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) __asm__ volatile("" : "+a"(bx[j]));
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        Pc[j] = mfma_e4m3_16x16x128(a[i], bx[j], zero);
        if (i > 0) fold(i - 1, j, Pp[j]);
      }
      if (i < kOpsPerBlock / 2) {
        issue_load(kb_pf, 2 * i, wnx, xnx);
        issue_load(kb_pf, 2 * i + 1, wnx, xnx);
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) fold(NI - 1, j, ((NI - 1) & 1) ? P1[j] : P0[j]);
    // instruction order: per MFMA one fold (4 VALU, 8 for Wgrad), and a DMA
    // after every second MFMA of the first rows
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i > 0) __builtin_amdgcn_sched_group_barrier(0x002, kLayout == kWgrad ? 8 : 4, 0);
        if ((j & 1) && i < kOpsPerBlock / 2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
  };

  // Prologue: blocks 0 and 1 (block 0 again when K has a single block), then
  // whole rounds of three steps with no conditions inside: K is padded to a
  // multiple of three blocks, and a padding step folds with scale 0 (its
  // partial sums come from a reload of the last block, so they are finite
  // unless a NaN has already reached the accumulator).  Every step issues the
  // same 14 DMA instructions, so one vmcnt threshold marks block kb landed,
  // and the compiler's wait tracking sees that the stage being read is the
  // one that has landed.
  issue_loads(0, lds_w0, lds_x0);
  issue_loads(KB > 1 ? 1 : 0, lds_w1, lds_x1);
  for (int kb = 0; kb < KB; kb += 3) {
    step(kb, lds_w0, lds_x0, lds_w2, lds_x2);
    step(kb + 1, lds_w1, lds_x1, lds_w0, lds_x0);
    step(kb + 2, lds_w2, lds_x2, lds_w1, lds_x1);
  }
  // the last step's reload DMA must land before the workgroup's LDS is released
  wait_vm_lgkm0<0>();

  // ---- epilogue: round and store ----
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int64_t m = m0 + wm * WM + j * 16 + lrow;
    if (m >= m_end) continue;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int64_t n = n0 + wn * WN + i * 16 + lgrp * 4;
      if (n >= p.N) continue;
      store4<kOutF32>(p, m, n, acc[i][j]);
    }
  }
}


// ---------------------------------------------------------------------------
// Direct-weight kernel (Fprop, Dgrad from W_q^T, Wgrad, grouped Fprop).
//
// Each wave owns 64 output columns (n) x all 128 token rows (m) of the
// 256 x 128 workgroup tile.  Its weight-side rows are private, so they skip
// LDS: they are loaded from memory straight into registers in MFMA operand
// layout, four K blocks deep.  Only the token-side tile, shared by the four
// waves, goes through LDS (four stages, DMA).  Per K step and CU this moves
// 80 KB through LDS (16 KB DMA writes + 64 KB operand reads) and 49 KB through
// the vector-memory unit, both below the 32 MFMAs per wave of the step.  The
// launch is persistent (one workgroup per CU walking its XCD's tiles) and
// full tiles store whole output row segments through an LDS staging area.
//
// k order inside an operand register: lane group g (= lane / 16) holds bytes
// 16g..16g+15 and 64+16g..64+16g+15 of the 128-byte K block (two aligned
// 64-byte halves per load instruction).  Both operands use the same order, so
// the MFMA contracts the same 128 products; each aligned run of 8 k stays
// together inside the MFMA.
// ---------------------------------------------------------------------------
constexpr int DNI = 4, DNJ = 8;                // wave tile: 64 (n) x 128 (m)
constexpr int kDStage = BM * BK;               // token tile per stage: 16 KB
// per-stage scales, an LDS object of their own so that the four tile stages
// fill the first 64 KB and every operand read takes an immediate offset from
// one base address
constexpr int kDScaleOff = 0;                  // token-side scales, [lrow][j] order (512 B)
constexpr int kDFreeOff = 512;                 // 512 B no DMA writes
constexpr int kDWScaleOff = 1024;              // weight-side scales (Wgrad: 256 per-column floats)
constexpr int kDScaleStage = 2048;
constexpr int kDOutStage = 16384;              // epilogue staging per wave: 128 x 64 BF16 or 64 x 64 FP32
constexpr int kDWOps = 8;                      // weight loads per block

template <int kLayout, bool kOutF32, bool kGrouped, bool kTiledB>
__global__ __launch_bounds__(kThreads, 1) void block_gemm_direct_kernel(GemmProblem p, int64_t total_tiles) {
  static_assert(kLayout != kDgrad, "Dgrad reads the weights transposed through LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a0[kDStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a1[kDStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a2[kDStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a3[kDStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_c0[kDScaleStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_c1[kDScaleStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_c2[kDScaleStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_c3[kDScaleStage];
  // per-wave epilogue staging, four objects of the stage size (one 64 KB
  // array would be placed first and push the tile stages past the 64 KB
  // reach of LDS instruction offsets)
  __shared__ __attribute__((aligned(1024))) uint8_t lds_z0[kDOutStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_z1[kDOutStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_z2[kDOutStage];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_z3[kDOutStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15, lgrp = lane >> 4;
  // stage k: token tile in lds_ak, its scales in lds_ck (k a compile-time tag)
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  auto tile_of = [&](auto k) -> uint8_t* {
    constexpr int s_ = decltype(k)::value;
    if constexpr (s_ == 0) return lds_a0;
    else if constexpr (s_ == 1) return lds_a1;
    else if constexpr (s_ == 2) return lds_a2;
    else return lds_a3;
  };
  auto scl_of = [&](auto k) -> uint8_t* {
    constexpr int s_ = decltype(k)::value;
    if constexpr (s_ == 0) return lds_c0;
    else if constexpr (s_ == 1) return lds_c1;
    else if constexpr (s_ == 2) return lds_c2;
    else return lds_c3;
  };
  // the same stages as LDS-address-space pointers, for the DMA destinations
  // (a cast of a generic pointer would carry a null check into M0)
  using lds_u8 = __attribute__((address_space(3))) uint8_t;
  auto tile_lds = [&](auto k) -> lds_u8* { return (lds_u8*)tile_of(k); };
  auto scl_lds = [&](auto k) -> lds_u8* { return (lds_u8*)scl_of(k); };

  // Persistent: the workgroup takes work ids blockIdx.x, + gridDim.x, ...;
  // each tile's last round streams the next tile's first blocks, so the
  // tile's stores overlap them.
  // Ids below plan.dp_tiles are whole tiles (gridDim.x is a multiple of 8,
  // so all of a workgroup's tiles lie in the same XCD's run); the ids after
  // them are the K pieces of the leftover tiles, one per workgroup, summed by
  // the piece that finishes last.
  const int KB = (int)(p.K / BK);
  // The schedule sits in LDS (stage 2's free scale bytes, one copy per wave)
  // and is read back at each tile boundary: registers held across the K loop
  // are scarce, and a grouped launch's extra state would otherwise spill.
  struct PlanLds {
    int64_t dp_tiles, split_tiles, work_ids;
    int32_t split, rounds;
  };
  static_assert(4 * sizeof(PlanLds) <= kDWScaleOff - kDFreeOff, "schedule fits the free scale bytes");
  PlanLds* plan_lds = reinterpret_cast<PlanLds*>(lds_c2 + kDFreeOff) + wave;
  // grouped launches of up to kLdsGroups groups: the group table in the free
  // scale bytes of stages 1 (first tiles) and 3 (row ranges), which no DMA
  // writes
  static_assert((kLdsGroups + 1) * 4 <= kDWScaleOff - kDFreeOff && 2 * kLdsGroups * 4 <= kDWScaleOff - kDFreeOff,
                "group table fits the free scale bytes");
  const GroupLds gtab{reinterpret_cast<int32_t*>(lds_c1 + kDFreeOff), reinterpret_cast<int32_t*>(lds_c3 + kDFreeOff),
                      reinterpret_cast<int32_t*>(lds_c3 + kDFreeOff) + kLdsGroups};
  const bool group_lds = kGrouped && p.groups <= kLdsGroups;
  if (group_lds) {
    if (wave == 0) build_group_lds(p, gtab, lane);
    __syncthreads();
  }
  {
    const int64_t n_tiles =
        kGrouped ? (group_lds ? (int64_t)gtab.cum[p.groups] : uniform_i64(grouped_tile_count(p))) : total_tiles;
    const SplitPlan pl = split_plan(n_tiles, gridDim.x, KB, p.ws_partial != nullptr ? p.ws_slots : 0);
    if (lane == 0)
      *plan_lds = PlanLds{pl.dp_tiles, pl.split_tiles, pl.dp_tiles + pl.split_tiles * pl.split, pl.split, pl.rounds};
  }
  auto load_plan = [&](int64_t& work_ids) -> SplitPlan {
    const PlanLds v = *plan_lds;
    work_ids = uniform_i64(v.work_ids);
    return SplitPlan{uniform_i64(v.dp_tiles), uniform_i64(v.split_tiles), __builtin_amdgcn_readfirstlane(v.split),
                     __builtin_amdgcn_readfirstlane(v.rounds)};
  };
  int kb_lo = 0, kb_hi = KB;        // the tile's K blocks
  int piece_slot = -1;              // split piece: its workspace slot; -1: a whole tile
  constexpr bool kBlockW = kLayout == kFprop || kLayout == kDgradT;
  // DMA per block: 4 token-row instructions, the token-side scales and the
  // weight-side scales; then the 8 weight loads
  constexpr int kDDmaOps = 6;
  constexpr int kDOpsPerBlock = kDDmaOps + kDWOps;
  int64_t m0 = 0, m_end = 0, n0 = 0;
  const uint8_t* Bp = p.B;
  const float* sBp = p.sB;
  int rows_m = 0, rows_n = 0;
  __amdgpu_buffer_rsrc_t rsrc_x, rsrc_w, rsrc_sw;
  uint32_t sw_off = 0;
  const float* sa_tile = p.sA;      // token-side scales of the tile's rows, block 0
  const float* sb_tile = p.sB;      // Wgrad: weight-side scales of the tile's columns, block 0
  // the same for the workgroup's next work item, decoded while the current
  // one runs so that its last round can stream the next tile's first blocks
  int nx_kb_lo = 0, nx_kb_hi = KB, nx_piece = -1, nx_rows_m = 0, nx_rows_n = 0;
  int64_t nx_m0 = 0, nx_m_end = 0, nx_n0 = 0;
  __amdgpu_buffer_rsrc_t nx_rsrc_x, nx_rsrc_w, nx_rsrc_sw;
  uint32_t nx_sw_off = 0;
  const float* nx_sa = p.sA;
  const float* nx_sb = p.sB;
  const uint32_t sa_kbytes = (uint32_t)p.ld_sa * 4u, sb_kbytes = (uint32_t)p.ld_sb * 4u;
  // token-side tile: rows m0.., DMA'd 8 rows x 128 B per instruction, 16-byte
  // chunks XOR-swizzled by row & 7 (row & 7 == (lane >> 3) & 7 here)
  const int xrow = wave * 32 + (lane >> 3);
  const uint32_t off_x = (uint32_t)(xrow * (int)p.lda + (((lane & 7) ^ (lane >> 3)) << 4));
  // token-scale DMA: lane l of wave w fetches the scale of row 16 j + lrow
  // for LDS float t = 64 (w & 1) + l = 8 lrow + j
  const int sc_t = 64 * (wave & 1) + lane;
  const uint32_t sc_row_off = (uint32_t)(((sc_t & 7) * 16 + (sc_t >> 3)) * 4);
  // weight-side rows n0 + 64 wave + 16 i + lrow, loaded straight into
  // registers; row-major: lane reads 16 B of its row; operand-tiled (ldb ==
  // K): the wave's 16-row groups are 2 KB tiles per K block, each half one
  // 1 KB run
  const uint32_t off_w = kTiledB ? (uint32_t)(wave * 4 * KB * 2048 + lane * 16)
                                 : (uint32_t)((wave * 64 + lrow) * (int)p.ldb + lgrp * 16);
  const uint32_t w_istride = kTiledB ? (uint32_t)(KB * 2048) : (uint32_t)(16 * p.ldb);
  const uint32_t w_hstride = kTiledB ? 1024u : 64u;
  const uint32_t w_kstride = kTiledB ? 2048u : (uint32_t)BK;
  // weight-side scales: Fprop / Dgrad_T - the wave's 128x128 weight block
  // (every lane fetches the same float; Fprop's table is [N/128][K/128],
  // Dgrad_T reads the forward table [K/128][N/128]); Wgrad - the workgroup's
  // 256 per-column scales
  const int64_t sw_elems = kLayout == kFprop ? (p.N / 128) * p.ld_sb
                                             : (kLayout == kDgradT ? (p.K / BK) * p.ld_sb : 0);
  const uint32_t sw_kstride = kLayout == kFprop ? 4u : (uint32_t)p.ld_sb * 4u;
  // decode work id `id` into the next-tile state and set up its buffer
  // resources; false if it names no tile
  auto setup_tile = [&](int64_t id) -> bool {
    int64_t work_ids;
    const SplitPlan plan = load_plan(work_ids);
    int64_t b;
    if (id < plan.dp_tiles) {
      b = xcd_remap(id, plan.dp_tiles);
      nx_kb_lo = 0;
      nx_kb_hi = KB;
      nx_piece = -1;
    } else {
      // pieces in K-range-major order, each XCD a contiguous run of them: an
      // XCD's pieces share one K range and neighbouring tiles, so its L2
      // serves the token rows and weight columns they have in common
      const int64_t pieces = plan.split_tiles * plan.split;
      const int q = (int)xcd_remap(id - plan.dp_tiles, pieces);
      const int range = q / (int)plan.split_tiles, t = q % (int)plan.split_tiles;
      b = plan.dp_tiles + t;
      int lo, hi;
      split_range(plan, range, KB, lo, hi);
      nx_kb_lo = __builtin_amdgcn_readfirstlane(lo);
      nx_kb_hi = __builtin_amdgcn_readfirstlane(hi);
      // the tile's partials lie together, in piece order
      nx_piece = __builtin_amdgcn_readfirstlane(t * plan.split + range);
    }
    int64_t tm0, tm_end, tn0;
    if (group_lds ? !decode_tile_lds(p, gtab, lane, b, tm0, tm_end, tn0, Bp, sBp)
                  : !decode_tile_index(p, kGrouped, b, tm0, tm_end, tn0, Bp, sBp))
      return false;
    nx_m0 = uniform_i64(tm0);
    nx_m_end = uniform_i64(tm_end);
    nx_n0 = uniform_i64(tn0);
    Bp = uniform_ptr(Bp);
    sBp = uniform_ptr(sBp);
    nx_rows_m = (int)(nx_m_end - nx_m0 < BM ? nx_m_end - nx_m0 : BM);
    nx_rows_n = (int)(p.N - nx_n0 < BN ? p.N - nx_n0 : BN);
    nx_rsrc_x = __builtin_amdgcn_make_buffer_rsrc((void*)(p.A + nx_m0 * p.lda), (short)0, nx_rows_m * (int)p.lda,
                                                  (int)kRsrcWord3);
    nx_rsrc_w = __builtin_amdgcn_make_buffer_rsrc((void*)(Bp + nx_n0 * p.ldb), (short)0, nx_rows_n * (int)p.ldb,
                                                  (int)kRsrcWord3);
    nx_rsrc_sw = __builtin_amdgcn_make_buffer_rsrc((void*)sBp, (short)0, (int)(sw_elems * 4), (int)kRsrcWord3);
    const int64_t nbw = (nx_n0 + 64 * wave) / 128;
    nx_sw_off = kLayout == kFprop ? (uint32_t)(nbw * p.ld_sb) * 4u : (uint32_t)nbw * 4u;
    nx_sa = p.sA + nx_m0;
    nx_sb = sBp + nx_n0;
    return true;
  };
  // the next-tile state becomes the current one
  auto adopt_next = [&]() {
    kb_lo = nx_kb_lo;
    kb_hi = nx_kb_hi;
    piece_slot = nx_piece;
    m0 = nx_m0;
    m_end = nx_m_end;
    n0 = nx_n0;
    rows_m = nx_rows_m;
    rows_n = nx_rows_n;
    rsrc_x = nx_rsrc_x;
    rsrc_w = nx_rsrc_w;
    rsrc_sw = nx_rsrc_sw;
    sw_off = nx_sw_off;
    sa_tile = nx_sa;
    sb_tile = nx_sb;
  };
  int64_t tile = blockIdx.x;
  {
    int64_t work_ids;
    (void)load_plan(work_ids);
    while (tile < work_ids && !setup_tile(tile)) tile += gridDim.x;
    if (tile >= work_ids) return;
    adopt_next();
  }

  auto this_rsrc_x = [&]() { return rsrc_x; };
  auto this_rsrc_w = [&]() { return rsrc_w; };
  auto this_rsrc_sw = [&]() { return rsrc_sw; };
  auto this_sw_off = [&]() { return sw_off; };
  auto this_sa = [&]() { return sa_tile; };
  auto this_sb = [&]() { return sb_tile; };
  auto this_rows_m = [&]() { return rows_m; };
  auto this_rows_n = [&]() { return rows_n; };
  // kNext: the load belongs to the next work item (its first blocks, streamed
  // by the current tile's last round)
  auto issue_load = [&](int kb, int op, auto stage, v8i (&wr)[DNI], auto next_tag) {
    constexpr bool kNext = decltype(next_tag)::value;
    lds_u8* st = tile_lds(stage);
    lds_u8* sc = scl_lds(stage);
    const __amdgpu_buffer_rsrc_t rsrc_x = kNext ? nx_rsrc_x : this_rsrc_x();
    const __amdgpu_buffer_rsrc_t rsrc_w = kNext ? nx_rsrc_w : this_rsrc_w();
    const __amdgpu_buffer_rsrc_t rsrc_sw = kNext ? nx_rsrc_sw : this_rsrc_sw();
    const uint32_t sw_off = kNext ? nx_sw_off : this_sw_off();
    const float* sa_tile = kNext ? nx_sa : this_sa();
    const float* sb_tile = kNext ? nx_sb : this_sb();
    const int rows_m = kNext ? nx_rows_m : this_rows_m();
    const int rows_n = kNext ? nx_rows_n : this_rows_n();
    // the per-step part of an address in the vector offset (one add per step,
    // shared by the step's loads), the per-load constant in the scalar offset;
    // the range check sees their sum, as before
    if (op < 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_x, (lds_ptr_t)(st + (wave * 4 + op) * 1024), 16,
                                               off_x + (uint32_t)(kb * BK), (uint32_t)(op * 8 * (int)p.lda), 0, 0);
    } else if (op == 4) {
      // The token-side scales of this block, rows m0..m0+127, land in LDS in
      // [lrow][j] order (float 8 lrow + j holds row 16 j + lrow) so a lane
      // reads its 8 scales as two 16-byte runs.  One float per lane: waves
      // 0 and 2 write floats 0..63, waves 1 and 3 floats 64..127 (identical
      // bytes).  32-bit block offset (validated: the scale tables stay below
      // 2^31 bytes) on a per-tile base keeps the resource cheap to rebuild.
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(reinterpret_cast<const uint8_t*>(sa_tile) + (uint32_t)kb * sa_kbytes), (short)0, rows_m * 4,
          (int)kRsrcWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(sc + kDScaleOff + 256 * (wave & 1)), 4,
                                               sc_row_off, 0, 0, 0);
    } else if (op == 5) {
      if constexpr (kLayout == kWgrad) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const uint8_t*>(sb_tile) + (uint32_t)kb * sb_kbytes), (short)0, rows_n * 4,
            (int)kRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(sc + kDWScaleOff), 16, (uint32_t)(lane * 16), 0, 0,
                                                 0);
      } else {
        // the wave's weight-block scale (every lane fetches the same float)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_sw, (lds_ptr_t)(sc + kDWScaleOff + wave * 256), 4,
                                                 sw_off + (uint32_t)kb * sw_kstride, 0, 0, 0);
      }
    } else {
      const int i = (op - kDDmaOps) >> 1, h = (op - kDDmaOps) & 1;
      const v4i v = __builtin_amdgcn_raw_buffer_load_b128(
          rsrc_w, off_w + (uint32_t)kb * w_kstride, (uint32_t)i * w_istride + (uint32_t)h * w_hstride, 0);
      wr[i][4 * h + 0] = v[0];
      wr[i][4 * h + 1] = v[1];
      wr[i][4 * h + 2] = v[2];
      wr[i][4 * h + 3] = v[3];
    }
  };

  // swizzled LDS addresses of this lane's token-side operand halves: row
  // 16 j + lrow (row & 7 == lrow & 7), bytes 16 lgrp.. and 64 + 16 lgrp..
  const int sw = lrow & 7;
  const int x_lo = lrow * 128 + ((lgrp ^ sw) << 4);
  const int x_hi = lrow * 128 + (((4 + lgrp) ^ sw) << 4);

  v4f acc[DNI][DNJ];
  v8i w0[DNI], w1[DNI], w2[DNI], w3[DNI];

  // ---- one K block per step: token tile in stage st, weights in wc ----
  // Issue order of the global loads: the token tile and scales of block kb+2
  // (DMA, rows 0-2), then the weights of block kb+3 (rows 3-6), in every
  // step.  After row kMid the wave waits for block kb+1 (its DMA was issued
  // in step kb-1 and only block kb+2's weights and this step's first
  // 2 (kMid + 1) loads came after it), passes the workgroup barrier, and
  // reads block kb+1's scales and first two token-side operand rows while
  // rows kMid+1.. of block kb still run on the matrix unit, so the next step
  // starts with its operands in registers.  The partial sums of a block's
  // last row are folded in the next step's first row.  Stage safety with four
  // stages: the DMA of step kb writes the stage of block kb-2, whose last
  // reads (step kb-2) every wave finished before the barrier of step kb-1.
  // (The compiler does not count the LDS-DMA instructions in its own waits
  // for the weight registers; with this order its stricter waits only cover
  // data that is needed by then anyway.)
  constexpr int kMid = 5;
  v8i bxa, bxb;                     // block kb+1: token-side operand rows 0, 1
  float tn[DNJ];                    // block kb+1: token-side scales
  float wn = 1.f;                   // block kb+1: weight-side block scale
  v4f Pl[DNI];                      // last row of partial sums of block kb-1
  float cl = 0.f;                   // and its scale
  auto zero_state = [&]() {
#pragma unroll
    for (int i = 0; i < DNI; ++i) {
#pragma unroll
      for (int j = 0; j < DNJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      Pl[i] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    cl = 0.f;
  };

  auto read_tn = [&](const uint8_t* scn, int half) {
    const float4 t = *reinterpret_cast<const float4*>(scn + kDScaleOff + lrow * 32 + half * 16);
    tn[4 * half + 0] = t.x;
    tn[4 * half + 1] = t.y;
    tn[4 * half + 2] = t.z;
    tn[4 * half + 3] = t.w;
  };
  auto prefetch = [&](auto stage) {
    const uint8_t* stn = tile_of(stage);
    const uint8_t* scn = scl_of(stage);
    if constexpr (kBlockW) wn = reinterpret_cast<const float*>(scn + kDWScaleOff)[wave * 64];
    read_tn(scn, 0);
    read_tn(scn, 1);
    bxa = pair(stn + x_lo, stn + x_hi);
    bxb = pair(stn + x_lo + 2048, stn + x_hi + 2048);
  };

  auto nx_clamp = [&](int b) { return b < nx_kb_hi ? b : nx_kb_hi - 1; };
  using cur_t = std::integral_constant<bool, false>;
  using nxt_t = std::integral_constant<bool, true>;
  // xj_tag: -1 in every round but a tile's last; there, the step's index j in
  // the tile's last round, whose loads past the tile's last block fetch the
  // next work item's first blocks instead (its DMA from step 2 on, its
  // weights from step 1 on) - the blocks its prologue would load, into the
  // same stages and registers
  auto step = [&](auto pad_tag, int kb, auto s_cur, v8i (&wc)[DNI], auto s_next, auto s_dma,
                  v8i (&wf)[DNI], auto xj_tag) {
    constexpr int XJ = decltype(xj_tag)::value;
    const uint8_t* st = tile_of(s_cur);
    const uint8_t* sc = scl_of(s_cur);
    const uint8_t* stn = tile_of(s_next);
    const uint8_t* scn = scl_of(s_next);
    constexpr bool kPad = decltype(pad_tag)::value;   // the round may hold padding steps
    const bool live = !kPad || kb < kb_hi;
    const int kb_d = kb + 2 < kb_hi ? kb + 2 : kb_hi - 1;   // token tile streamed this step
    const int kb_w = kb + 3 < kb_hi ? kb + 3 : kb_hi - 1;   // weights streamed this step

    // c[j] (this block's scale of token subtile j) is formed in row j and
    // first used in row j+1
    float c[DNJ];
    float4 rs[DNI];
    if constexpr (kLayout == kWgrad) {
      const float* swl = reinterpret_cast<const float*>(sc + kDWScaleOff);
#pragma unroll
      for (int i = 0; i < DNI; ++i)
        rs[i] = *reinterpret_cast<const float4*>(swl + wave * 64 + i * 16 + lgrp * 4);
    }
    auto fold = [&](v4f& a, const v4f& P, float cj, int i) {
      if constexpr (kLayout == kWgrad) {
        a[0] = __builtin_fmaf(P[0] * rs[i].x, cj, a[0]);
        a[1] = __builtin_fmaf(P[1] * rs[i].y, cj, a[1]);
        a[2] = __builtin_fmaf(P[2] * rs[i].z, cj, a[2]);
        a[3] = __builtin_fmaf(P[3] * rs[i].w, cj, a[3]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) a[v] = __builtin_fmaf(P[v], cj, a[v]);
      }
    };

    v4i bxl[DNJ], bxh[DNJ];           // token-side operand halves, read two rows ahead
    bxl[0] = lo_half(bxa); bxh[0] = hi_half(bxa);
    bxl[1] = lo_half(bxb); bxh[1] = hi_half(bxb);
    v4i an_l, an_h, bn_l, bn_h;       // block kb+1's first two operand rows
    // rows j of 4 MFMAs (the wave's 4 weight subtiles against token subtile
    // j), each MFMA followed by the fold of the same subtile's partial from
    // row j-1 (row 0: the previous block's last row).  The other work of a
    // row is spread one item per MFMA so that no gap between two MFMAs holds
    // more than the 28 issue cycles the matrix unit is busy: rows 0-5 read
    // the operand halves of row j+2 (MFMAs 0 and 2) and issue two loads
    // (MFMAs 1 and 3); row 5 ends with the wait and barrier for block kb+1,
    // whose operands and scales rows 6-7 read.
    v4f P0[DNI], P1[DNI];
    // the operands stay in whichever register file the allocator gave them
    // (the MFMA reads both); pinning them to AGPRs costs a copy per register
    // of every weight buffer that crosses the loop's back edge
#pragma unroll
    for (int j = 0; j < DNJ; ++j) {
      v4f (&Pc)[DNI] = (j & 1) ? P1 : P0;
      v4f (&Pp)[DNI] = (j & 1) ? P0 : P1;
      const v8i bj = join(bxl[j], bxh[j]);
#pragma unroll
      for (int i = 0; i < DNI; ++i) {
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        Pc[i] = mfma_e4m3_16x16x128(wc[i], bj, zero);
        __builtin_amdgcn_sched_barrier(0);
        if (j > 0) fold(acc[i][j - 1], Pp[i], c[j - 1], i);
        else if constexpr (kBlockW) fold(acc[i][DNJ - 1], Pl[i], cl, i);
        if (i == 1) {
          const float t = kBlockW ? tn[j] * wn : tn[j];
          c[j] = live ? t : 0.f;
        }
        if (j + 2 < DNJ) {
          if (i == 0) bxl[j + 2] = *reinterpret_cast<const v4i*>(st + x_lo + (j + 2) * 2048);
          if (i == 2) bxh[j + 2] = *reinterpret_cast<const v4i*>(st + x_hi + (j + 2) * 2048);
        }
        if ((i & 1) && 2 * j + (i >> 1) < kDOpsPerBlock) {
          const int op = 2 * j + (i >> 1);
          if constexpr (XJ < 0) {
            issue_load(op < kDDmaOps ? kb_d : kb_w, op, s_dma, wf, cur_t{});
          } else if (op < kDDmaOps) {
            if constexpr (XJ >= 2) issue_load(nx_clamp(nx_kb_lo + XJ - 2), op, s_dma, wf, nxt_t{});
            else issue_load(kb_d, op, s_dma, wf, cur_t{});
          } else {
            if constexpr (XJ >= 1) issue_load(nx_clamp(nx_kb_lo + XJ - 1), op, s_dma, wf, nxt_t{});
            else issue_load(kb_w, op, s_dma, wf, cur_t{});
          }
        }
        if (j == DNJ - 2) {
          if (i == 0) an_l = *reinterpret_cast<const v4i*>(stn + x_lo);
          if (i == 1) an_h = *reinterpret_cast<const v4i*>(stn + x_hi);
          if (i == 2) bn_l = *reinterpret_cast<const v4i*>(stn + x_lo + 2048);
          if (i == 3) bn_h = *reinterpret_cast<const v4i*>(stn + x_hi + 2048);
        }
        if (j == DNJ - 1) {
          // the next block's scales; tn[0..7] are consumed by this step's
          // rows before these reads (c[j] above), so they can be refilled
          if (i == 0) read_tn(scn, 0);
          if (i == 1) read_tn(scn, 1);
          if constexpr (kBlockW) {
            if (i == 2) wn = reinterpret_cast<const float*>(scn + kDWScaleOff)[wave * 64];
          }
        }
        // instruction order = source order: one MFMA, then the fold of the
        // partial it produced four MFMAs (20 instructions) earlier
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j == kMid) {
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<kDWOps + 2 * (kMid + 1)>();
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    bxa = join(an_l, an_h);
    bxb = join(bn_l, bn_h);
    if constexpr (kBlockW) {
#pragma unroll
      for (int i = 0; i < DNI; ++i) Pl[i] = ((DNJ - 1) & 1) ? P1[i] : P0[i];
      cl = c[DNJ - 1];
    } else {
#pragma unroll
      for (int i = 0; i < DNI; ++i) fold(acc[i][DNJ - 1], ((DNJ - 1) & 1) ? P1[i] : P0[i], c[DNJ - 1], i);
    }
  };

  // Prologue of the workgroup's first tile, in the steady-state order
  // (weights of its first block; tile of the first block and weights of the
  // second; tile of the second and weights of the third), blocks past the
  // tile's K range repeating its last block; later tiles get the same loads
  // from the previous tile's last round.  The wait at the top of each tile
  // allows the 22 loads issued after block 0's tile (any stores issued after
  // them are younger still), then block 0's first operands are read.  Whole
  // rounds of four steps follow with no conditions inside; when K is not a
  // multiple of four blocks the last round pads with steps that fold with
  // scale 0.
  auto issue_prologue = [&]() {
    auto clamp = [&](int b) { return b < kb_hi ? b : kb_hi - 1; };
#pragma unroll
    for (int op = kDDmaOps; op < kDOpsPerBlock; ++op) issue_load(kb_lo, op, S0{}, w0, cur_t{});
#pragma unroll
    for (int op = 0; op < kDDmaOps; ++op) issue_load(kb_lo, op, S0{}, w0, cur_t{});
#pragma unroll
    for (int op = kDDmaOps; op < kDOpsPerBlock; ++op) issue_load(clamp(kb_lo + 1), op, S1{}, w1, cur_t{});
#pragma unroll
    for (int op = 0; op < kDDmaOps; ++op) issue_load(clamp(kb_lo + 1), op, S1{}, w1, cur_t{});
#pragma unroll
    for (int op = kDDmaOps; op < kDOpsPerBlock; ++op) issue_load(clamp(kb_lo + 2), op, S2{}, w2, cur_t{});
  };
  // ---- epilogue: lane holds 4 consecutive n of row m for every (i, j) ----
  auto store_tile = [&](int64_t em0, int64_t em_end, int64_t en0, int erows_m, int erows_n) {
    if (erows_m == BM && erows_n == BN) {
      // Full tile: the wave's 64 (n) x 128 (m) block goes through its own
      // staging area so that every store instruction writes whole row segments
      // of the output: 8 rows x 128 B (BF16) or 4 rows x 256 B (FP32, in two
      // halves of 64 rows).  Lane stores of 4 values per row took ~2.5x as
      // long, all workgroups of a round storing at once.  16-byte chunks are
      // XOR-swizzled by row.  The output is written once and not read by the
      // kernel: non-temporal stores keep it from displacing operand lines
      // in the MALL (Fprop 446 -> 432 us and grouped 235 -> 228 us in
      // back-to-back launches, where the weights stay resident between
      // launches; inside a step whose other kernels evict them anyway, Fprop
      // 459 -> 455 us and grouped 255 -> 250 us).
      uint8_t* ob = wave == 0 ? lds_z0 : wave == 1 ? lds_z1 : wave == 2 ? lds_z2 : lds_z3;
      if constexpr (!kOutF32) {
#pragma unroll
        for (int j = 0; j < DNJ; ++j) {
#pragma unroll
          for (int i = 0; i < DNI; ++i) {
            const int m = j * 16 + lrow, nl = i * 16 + lgrp * 4;
            const v4f& r = acc[i][j];
            const __bf16 h0 = (__bf16)r[0], h1 = (__bf16)r[1], h2 = (__bf16)r[2], h3 = (__bf16)r[3];
            const uint32_t u0 = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
            const uint32_t u1 = (uint32_t)__builtin_bit_cast(uint16_t, h2) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
            *reinterpret_cast<uint2*>(ob + m * 128 + (((nl >> 3) ^ (m & 7)) << 4) + (nl & 7) * 2) =
                make_uint2(u0, u1);
          }
        }
#pragma unroll
        for (int t = 0; t < BM / 8; ++t) {
          const int row = t * 8 + (lane >> 3), ch = lane & 7;
          const v4i v = *reinterpret_cast<const v4i*>(ob + row * 128 + ((ch ^ (row & 7)) << 4));
          uint16_t* dst = reinterpret_cast<uint16_t*>(p.C) + (em0 + row) * p.ldc + en0 + wave * 64 + ch * 8;
          __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(dst));
        }
      } else {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int j = 0; j < DNJ / 2; ++j) {
#pragma unroll
            for (int i = 0; i < DNI; ++i) {
              const int m = j * 16 + lrow, ch = i * 4 + lgrp;
              const v4f& r = acc[i][half * (DNJ / 2) + j];
              *reinterpret_cast<float4*>(ob + m * 256 + ((ch ^ (m & 15)) << 4)) = make_float4(r[0], r[1], r[2], r[3]);
            }
          }
#pragma unroll
          for (int t = 0; t < BM / 8; ++t) {
            const int row = t * 4 + (lane >> 4), ch = lane & 15;
            const v4i v = *reinterpret_cast<const v4i*>(ob + row * 256 + ((ch ^ (row & 15)) << 4));
            float* dst = reinterpret_cast<float*>(p.C) + (em0 + half * (BM / 2) + row) * p.ldc + en0 + wave * 64 + ch * 4;
            __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(dst));
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < DNJ; ++j) {
        const int64_t m = em0 + j * 16 + lrow;
        if (m >= em_end) continue;
#pragma unroll
        for (int i = 0; i < DNI; ++i) {
          const int64_t n = en0 + wave * 64 + i * 16 + lgrp * 4;
          if (n >= p.N) continue;
          store4<kOutF32>(p, m, n, acc[i][j]);
        }
      }
    }
  };
  zero_state();
  issue_prologue();
  // Each work item decodes the next one first.  Its last round (padded
  // with scale-0 steps when the item's K blocks are not a multiple of four)
  // streams the next item's first blocks into the stages and registers the
  // prologue would use, so the item's stores overlap those loads and the
  // next item starts without a prologue.  A workgroup's last item streams
  // its own last block again instead (harmless reloads, drained at the end).
  for (;;) {
  wait_vm<kDDmaOps + 2 * kDWOps>();
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  int64_t next = tile + gridDim.x;
  bool more;
  {
    int64_t work_ids;
    (void)load_plan(work_ids);
    while (next < work_ids && !setup_tile(next)) next += gridDim.x;
    more = next < work_ids;
  }
  if (!more) {
    // no next item: its "first blocks" are this tile's last block
    nx_kb_lo = kb_hi - 1;
    nx_kb_hi = kb_hi;
    nx_rows_m = rows_m;
    nx_rows_n = rows_n;
    nx_rsrc_x = rsrc_x;
    nx_rsrc_w = rsrc_w;
    nx_rsrc_sw = rsrc_sw;
    nx_sw_off = sw_off;
    nx_sa = sa_tile;
    nx_sb = sb_tile;
  }
  prefetch(S0{});
  using no_pad = std::integral_constant<bool, false>;
  using pad = std::integral_constant<bool, true>;
  using xn = std::integral_constant<int, -1>;
  const int kb_last = kb_lo + ((kb_hi - kb_lo + 3) & ~3) - 4;   // first block of the last round
  int kb = kb_lo;
  for (; kb < kb_last; kb += 4) {
    step(no_pad{}, kb, S0{}, w0, S1{}, S2{}, w3, xn{});
    step(no_pad{}, kb + 1, S1{}, w1, S2{}, S3{}, w0, xn{});
    step(no_pad{}, kb + 2, S2{}, w2, S3{}, S0{}, w1, xn{});
    step(no_pad{}, kb + 3, S3{}, w3, S0{}, S1{}, w2, xn{});
  }
  step(pad{}, kb, S0{}, w0, S1{}, S2{}, w3, std::integral_constant<int, 0>{});
  step(pad{}, kb + 1, S1{}, w1, S2{}, S3{}, w0, std::integral_constant<int, 1>{});
  step(pad{}, kb + 2, S2{}, w2, S3{}, S0{}, w1, std::integral_constant<int, 2>{});
  step(pad{}, kb + 3, S3{}, w3, S0{}, S1{}, w2, std::integral_constant<int, 3>{});
  if constexpr (kBlockW) {
#pragma unroll
    for (int i = 0; i < DNI; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][DNJ - 1][v] = __builtin_fmaf(Pl[i][v], cl, acc[i][DNJ - 1][v]);
  }
  const int64_t em0 = m0, em_end = m_end, en0 = n0;
  const int erows_m = rows_m, erows_n = rows_n;
  const int epiece = piece_slot;
  int64_t work_ids;
  const SplitPlan plan = load_plan(work_ids);
  if (epiece >= 0) {
    // A K piece of a split tile (a workgroup's last work item).  Its FP32
    // partial tile goes to the workspace in fragment order (16 B per lane per
    // (i, j): 1 KB per wave per store); then the tile's counter counts it.
    // The piece that arrives last adds the tile's partials in piece order -
    // a fixed order, so the result does not depend on which piece that is -
    // zeroes the counter for the next launch, and stores the tile.
    constexpr int kWaveF4 = DNI * DNJ * 64;
    constexpr int64_t kTileF4 = kSplitTileFloats / 4;
    float4* part = reinterpret_cast<float4*>(p.ws_partial) + (int64_t)epiece * kTileF4 + wave * kWaveF4 + lane;
#pragma unroll
    for (int i = 0; i < DNI; ++i)
#pragma unroll
      for (int j = 0; j < DNJ; ++j)
        part[(i * DNJ + j) * 64] = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    // Release: each wave's partial stores are complete (acknowledged by its
    // XCD's L2) before the barrier - a workgroup barrier alone does not wait
    // for them - then one lane writes that L2's dirty lines back (so the
    // other XCDs see them) and counts the piece.  One fence per piece, not
    // one per wave: each writes back the whole L2.
    wait_vm_lgkm0<0>();
    __syncthreads();
    // the arrival count passes through unused bytes of stage 0 (no DMA is
    // in flight: a piece is its workgroup's last work item; a separate LDS
    // object would move the stages past the 64 KB reach of LDS offsets)
    uint32_t* arrive = reinterpret_cast<uint32_t*>(lds_c0 + kDFreeOff);
    const int et = epiece / plan.split;
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      *arrive = atomicAdd(&p.ws_count[et], 1u);
    }
    __syncthreads();
    if (*arrive != (uint32_t)(plan.split - 1)) return;
    // Acquire, by the wave that read the final count: drop stale lines from
    // the CU's L1 and the XCD's L2, which the whole workgroup shares, before
    // any wave reads the other pieces' partials
    if (wave == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
    // partial 0, then partials 1.. added in turn, each read as one batch of
    // 32 independent 16-byte loads per lane
    const float4* first = reinterpret_cast<const float4*>(p.ws_partial) + (int64_t)et * plan.split * kTileF4 +
                          wave * kWaveF4 + lane;
#pragma unroll
    for (int i = 0; i < DNI; ++i)
#pragma unroll
      for (int j = 0; j < DNJ; ++j) {
        const float4 u = first[(i * DNJ + j) * 64];
        acc[i][j] = v4f{u.x, u.y, u.z, u.w};
      }
    for (int q = 1; q < plan.split; ++q) {
      const float4* src = first + (int64_t)q * kTileF4;
      float4 u[DNI][DNJ];
#pragma unroll
      for (int i = 0; i < DNI; ++i)
#pragma unroll
        for (int j = 0; j < DNJ; ++j) u[i][j] = src[(i * DNJ + j) * 64];
#pragma unroll
      for (int i = 0; i < DNI; ++i)
#pragma unroll
        for (int j = 0; j < DNJ; ++j) {
          acc[i][j][0] += u[i][j].x;
          acc[i][j][1] += u[i][j].y;
          acc[i][j][2] += u[i][j].z;
          acc[i][j][3] += u[i][j].w;
        }
    }
    if (tid == 0) p.ws_count[et] = 0u;
    // the split path ends here and never reaches the K loop again (the
    // compiler's wait analysis would otherwise carry its loads into the loop)
    store_tile(em0, em_end, en0, erows_m, erows_n);
    return;
  }
  store_tile(em0, em_end, en0, erows_m, erows_n);
  if (!more) {
    wait_vm<0>();   // the reloads streamed by the last round land before the workgroup ends
    break;
  }
  adopt_next();
  tile = next;
  zero_state();
  }
}

template <int kLayout, bool kGrouped>
hipError_t launch_typed(const GemmProblem& p, hipStream_t stream, int64_t grid, int64_t total) {
  if constexpr (kLayout == kDgrad) {
    if (p.out_fp32) {
      hipLaunchKernelGGL((block_gemm_kernel<kLayout, true, kGrouped>), dim3((unsigned)grid),
                         dim3(kThreads), 0, stream, p, total);
    } else {
      hipLaunchKernelGGL((block_gemm_kernel<kLayout, false, kGrouped>), dim3((unsigned)grid),
                         dim3(kThreads), 0, stream, p, total);
    }
  } else {
    grid = persistent_grid(grid);
    if (p.b_tiled) {
      if (p.out_fp32) {
        hipLaunchKernelGGL((block_gemm_direct_kernel<kLayout, true, kGrouped, true>), dim3((unsigned)grid),
                           dim3(kThreads), 0, stream, p, total);
      } else {
        hipLaunchKernelGGL((block_gemm_direct_kernel<kLayout, false, kGrouped, true>), dim3((unsigned)grid),
                           dim3(kThreads), 0, stream, p, total);
      }
    } else {
      if (p.out_fp32) {
        hipLaunchKernelGGL((block_gemm_direct_kernel<kLayout, true, kGrouped, false>), dim3((unsigned)grid),
                           dim3(kThreads), 0, stream, p, total);
      } else {
        hipLaunchKernelGGL((block_gemm_direct_kernel<kLayout, false, kGrouped, false>), dim3((unsigned)grid),
                           dim3(kThreads), 0, stream, p, total);
      }
    }
  }
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device (cached); 0 if unknown.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 0;
  }
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      return 0;
    }
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups of a persistent direct-kernel launch over `ids` tiles: one per
// CU (the LDS footprint allows no second one), a multiple of 8 so that each
// workgroup stays on one XCD's tile run; one per tile when there are fewer.
int64_t persistent_grid(int64_t ids) {
  const int cus = device_cus();
  return (cus >= 8 && ids > cus) ? cus / 8 * 8 : ids;
}

// ---- split workspace for callers that cannot allocate ----
// One partial tile per piece for kStaticSlots pieces (one per CU of a
// device with up to kStaticSlots CUs), then the per-tile counters: 32 MB +
// 1 KB, held by every GPU the library runs on until the process ends.  In
// host code `scratch` only stands for the symbol; its device address comes
// from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kStaticSlots * kSplitTileFloats * 4 + kStaticSlots * 4];

__global__ void zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t attach_static_workspace(GemmProblem& p, hipStream_t stream) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* base[kMaxDev];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  const size_t count_off = (size_t)kStaticSlots * (size_t)kSplitTileFloats * 4u;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (base[dev] == nullptr) {
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      // the counters start at zero (each launch leaves them zero); cleared
      // by a kernel, not a memset, so that a capturing caller records a
      // kernel node
      hipLaunchKernelGGL(zero_words, dim3(1), dim3(kStaticSlots), 0, stream,
                         reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ptr) + count_off), (int)kStaticSlots);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      base[dev] = ptr;
    }
    p.ws_partial = static_cast<float*>(base[dev]);
    p.ws_count = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(base[dev]) + count_off);
    p.ws_slots = kStaticSlots;
  }
  return hipSuccess;
}

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
    case kDgradT: return launch_typed<kDgradT, false>(p, stream, total, total);
    default: return launch_typed<kWgrad, false>(p, stream, total, total);
  }
}

}  // namespace fp8bs
