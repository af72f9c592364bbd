/*
 * fp8bs.h - fine-grained FP8 (E4M3) block-scaled quantization and GEMM for
 * AMD MI355X (gfx950).  C ABI of libfp8bs.so.
 *
 * What the library computes (sources are the pages' titles and sections):
 *
 *  - Online activation quantization with one FP32 scale per 1x128 tile of
 *    contiguous channels of one token ("Fine-Grained FP8 Quantization in
 *    DeepSeek", section 2; "FP8 Mixed Precision: DeepSeek-V3 Training
 *    Architecture", section 1 item 1; "Introduction to LLM Quantization",
 *    section 5).
 *  - Weight quantization with one FP32 scale per 128x128 block ("Fine-Grained
 *    FP8 Quantization in DeepSeek", section 3; "FP8 Mixed Precision:
 *    DeepSeek-V3 Training Architecture", section 1 item 2 and its block-scale
 *    equations).
 *  - Block-scaled FP8 GEMM: E4M3 products accumulated in FP32, each 128-wide
 *    K block's partial sum multiplied by its two scales, blocks summed in
 *    FP32, result rounded once to BF16 (or kept FP32) ("FP8 Mixed Precision:
 *    DeepSeek-V3 Training Architecture", section 3 "Decoupled Accumulation in
 *    Tensor Core GEMMs"; "Fine-Grained FP8 Quantization in DeepSeek", section
 *    4; "Introduction to LLM Quantization", section 2 steps 1-4), in the
 *    forward (Fprop),
 *    input-gradient (Dgrad) and weight-gradient (Wgrad) layouts
 *    ("Introduction to LLM Quantization", section 1 items 2-3).
 *
 * Quantization rule, per tile (bit-exact, no FMA contraction, no flush of
 * denormals):
 *     amax = max |x|                       (x: BF16 widened exactly to FP32)
 *     s    = max(fl32(amax / 448), fl32(1e-12))
 *     q    = E4M3(fl32(x / s))             (true IEEE division)
 *  E4M3 is the 1-4-3 format with bias 7, largest finite 448, no infinities and
 *  NaN = S.1111.111.  The cast rounds to nearest, ties to even, and saturates
 *  finite overflow and +-Inf to +-448; a NaN quotient becomes code 0x7F.  A
 *  tile containing NaN gets scale 0x7FC00000 (canonical NaN) and all-NaN
 *  codes; a tile containing +-Inf gets scale +Inf.  The stored scale is the
 *  dequantization multiplier s (x ~ decode(q) * s).
 *
 * Conventions for every entry point:
 *  - All matrices are row-major; ld* are leading dimensions in ELEMENTS.
 *  - Every pointer except the host-side ones named below is a DEVICE pointer
 *    allocated by the caller.  The library never allocates, frees or
 *    synchronizes; it keeps no state beyond per-device properties it caches
 *    on first use.  Entry points are thread-safe.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued asynchronously on it; faults during execution surface at
 *    the caller's next synchronization, as in HIP.
 *  - Arguments are validated on the host before anything is launched; on any
 *    error nothing is launched and the status says why.  No exceptions cross
 *    the ABI.
 *  - Alignment: FP8/BF16/FP32 matrix base pointers must be 16-byte aligned and
 *    every row start must be 16-byte aligned (ld * element size % 16 == 0);
 *    scale arrays need 4-byte alignment.
 *  - Calls that overlap on one stream are ordered; calls on different streams
 *    that write the same buffers race.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8BS_ABI_VERSION 1

typedef enum {
  FP8_OK = 0,
  FP8_ERR_NULL = 1,        /* a required pointer is NULL */
  FP8_ERR_SHAPE = 2,       /* negative size, or a dimension not a multiple of 128 where required */
  FP8_ERR_LD = 3,          /* leading dimension smaller than the row length */
  FP8_ERR_ALIGN = 4,       /* pointer or row stride not 16-byte aligned */
  FP8_ERR_UNSUPPORTED = 5, /* unknown enum value or unsupported combination */
  FP8_ERR_DEVICE = 6,      /* no current HIP device, or it is not gfx950 */
  FP8_ERR_LAUNCH = 7,      /* the kernel launch itself failed */
  FP8_ERR_ALIAS = 8        /* an output buffer overlaps an input buffer */
} fp8_status;

typedef enum {
  FP8_TILE_ROW = 0, /* 1x128 tiles along the columns of each row */
  FP8_TILE_COL = 1, /* 128x1 tiles along the rows of each column; output transposed */
  FP8_TILE_COL_TILED = 2 /* FP8_TILE_COL with the transposed codes written operand-tiled */
} fp8_tile_dir;

typedef enum {
  FP8_LAYOUT_FPROP = 0, /* C[M][N] = A[M][K] . B[N][K]^T,  B = W_q (weights [d_out][d_in]) */
  FP8_LAYOUT_DGRAD = 1, /* C[M][N] = A[M][K] . B[K][N],    B = W_q stored [d_out = K][d_in = N] */
  FP8_LAYOUT_WGRAD = 2, /* C[M][N] = A[M][K] . B[N][K]^T,  K = tokens, per-row x per-column scales */
  FP8_LAYOUT_DGRAD_T = 3, /* C[M][N] = A[M][K] . B[N][K]^T,  B = W_q^T (transposed weight codes) */
  FP8_LAYOUT_FPROP_TILED = 4,  /* FPROP with B in the operand-tiled layout (ldb == K) */
  FP8_LAYOUT_DGRAD_T_TILED = 5, /* DGRAD_T with B in the operand-tiled layout (ldb == K) */
  FP8_LAYOUT_WGRAD_TILED = 6    /* WGRAD with B = X_q^T in the operand-tiled layout (ldb == K) */
} fp8_gemm_layout;

typedef enum { FP8_OUT_BF16 = 0, FP8_OUT_FP32 = 1 } fp8_out_dtype;

/*
 * fp8_quant_act_1x128 - online activation quantization (see the rule above).
 *
 *  x          BF16 [rows][ldx >= cols]
 *  dir        FP8_TILE_ROW: tiles of 1x128 along each row; requires cols % 128 == 0.
 *               q      [rows][ldq >= cols]            E4M3 codes
 *               scales [cols/128][ld_s >= rows]       FP32, MN-major: the scales of
 *                                                     one K block are contiguous
 *                                                     over rows, matching the
 *                                                     GEMM's A-scale layout
 *             FP8_TILE_COL: tiles of 128x1 along each column (weight-gradient
 *             operands, tiles along tokens); requires rows % 128 == 0.
 *             FP8_TILE_COL_TILED: the same codes written in the operand-tiled
 *             layout of fp8_quant_weight_128x128_tiled (R = cols, C = rows),
 *             for FP8_LAYOUT_WGRAD_TILED; also cols % 128 == 0 and ldq == rows.
 *               q      [cols][ldq >= rows]            transposed codes (K-contiguous
 *                                                     for the Wgrad GEMM)
 *               scales [rows/128][ld_s >= cols]       FP32
 *  scales_in  NULL: online scales from each tile's amax, written to `scales`.
 *             Otherwise caller-supplied scales (same layout as `scales`; used
 *             by delayed / history / fixed scale policies): codes are
 *             E4M3(fl32(x / s_in)) and `scales` is not written (may be NULL).
 *             ROW direction only.
 *  amax_out   optional (NULL): per-tile max |x| in the scale layout
 *             (canonical NaN for tiles containing NaN).
 *  sat_count  optional (NULL) device uint32 counter, incremented atomically by
 *             the number of elements the saturating cast clips
 *             (|fl32(x / s)| > 464, Inf included, NaN not).  The caller zeroes
 *             it.  Online scales never clip.
 *  rows == 0 or cols == 0 is a no-op returning FP8_OK.
 */
fp8_status fp8_quant_act_1x128(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                               fp8_tile_dir dir, uint8_t* q, int64_t ldq,
                               float* scales, int64_t ld_s, const float* scales_in,
                               float* amax_out, uint32_t* sat_count, void* stream);

/*
 * fp8_quant_act_dual - both orientations of a backward-pass activation from
 * one read of it: the 1x128 row tiles that Dgrad consumes and the 128x1
 * column tiles, transposed, that Wgrad consumes.  The outputs are exactly
 * those of fp8_quant_act_1x128 with FP8_TILE_ROW and with FP8_TILE_COL
 * (online scales).  One read of x instead of two ("Online Quantization
 * During Training" section 5: separate passes move the tensor through memory
 * again and again; "Fine-Grained FP8 Quantization in DeepSeek" section 4:
 * the transpose layout decides real performance).
 *
 *  x      BF16 [rows][ldx >= cols]; rows % 128 == 0 and cols % 128 == 0.
 *  q_row  [rows][ldq_row >= cols]          row-tile codes
 *  s_row  [cols/128][ld_s_row >= rows]     row-tile scales (MN-major)
 *  q_col  [cols][ldq_col >= rows]          column-tile codes, transposed
 *  s_col  [rows/128][ld_s_col >= cols]     column-tile scales
 *  No output may overlap x or another output.
 */
fp8_status fp8_quant_act_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                              uint8_t* q_row, int64_t ldq_row, float* s_row, int64_t ld_s_row,
                              uint8_t* q_col, int64_t ldq_col, float* s_col, int64_t ld_s_col,
                              void* stream);

/* fp8_quant_act_dual_tiled - fp8_quant_act_dual with the column-tile codes
 * written operand-tiled (dense, cols * rows bytes; see FP8_TILE_COL_TILED). */
fp8_status fp8_quant_act_dual_tiled(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                    uint8_t* q_row, int64_t ldq_row, float* s_row, int64_t ld_s_row,
                                    uint8_t* q_col_tiled, float* s_col, int64_t ld_s_col,
                                    void* stream);

/*
 * fp8_quant_weight_128x128 - 128x128 weight-block quantization, blocks
 * anchored at (0, 0); same per-block rule as above over 16384 values.
 *
 *  w       BF16 [rows][ldw >= cols]; rows % 128 == 0 and cols % 128 == 0.
 *  q       E4M3 [rows][ldq >= cols]
 *  q_t     optional (NULL): the same codes transposed, [cols][ldq_t >= rows]
 *  scales  FP32 [rows/128][ld_s >= cols/128]
 */
fp8_status fp8_quant_weight_128x128(const void* w, int64_t rows, int64_t cols, int64_t ldw,
                                    uint8_t* q, int64_t ldq, uint8_t* q_t, int64_t ldq_t,
                                    float* scales, int64_t ld_s, void* stream);

/*
 * fp8_quant_weight_128x128_tiled - the same quantization with the codes
 * written in the operand-tiled layout the GEMM's *_TILED layouts read
 * ("Fine-Grained FP8 Quantization in DeepSeek", section 4: how operands and
 * their scales are laid out decides real performance).  For a code matrix
 * Q [R][C] the tiled array holds R * C bytes; element (r, c) is at
 *     ((r / 16) * (C / 128) + c / 128) * 2048 + ((c % 128) / 64) * 1024
 *       + (((c % 64) / 16) * 16 + r % 16) * 16 + c % 16
 * so every 1 KB half of a 2 KB tile is one contiguous 16-byte-per-lane load
 * of a wave.  The codes and scales equal fp8_quant_weight_128x128's.
 *  q_tiled    [rows * cols] bytes: W_q tiled (R = rows, C = cols)
 *  q_t_tiled  optional (NULL): W_q^T tiled (R = cols, C = rows), for
 *             FP8_LAYOUT_DGRAD_T_TILED
 *  scales     FP32 [rows/128][ld_s >= cols/128]
 */
fp8_status fp8_quant_weight_128x128_tiled(const void* w, int64_t rows, int64_t cols, int64_t ldw,
                                          uint8_t* q_tiled, uint8_t* q_t_tiled, float* scales,
                                          int64_t ld_s, void* stream);

/*
 * fp8_block_gemm - block-scaled FP8 GEMM, FP32 accumulation, per-128-K scale
 * epilogue:
 *     C[m][n] = round( sum_kb  sa(m, kb) * sb(n, kb) * sum_{k in kb} A(m, k) * B(k, n) )
 *  K is always the contraction dimension and K % 128 == 0, K > 0.
 *
 *  FP8_LAYOUT_FPROP   (M = tokens, N = d_out, K = d_in)
 *     A  = X_q  [M][lda >= K];     sA [K/128][ld_sa >= M]     (1x128 row scales)
 *     B  = W_q  [N][ldb >= K];     sB [N/128][ld_sb >= K/128] (128x128 block scales)
 *     N % 128 == 0.
 *  FP8_LAYOUT_DGRAD   (M = tokens, N = d_in, K = d_out)
 *     A  = dY_q [M][lda >= K];     sA [K/128][ld_sa >= M]     (1x128 row scales)
 *     B  = W_q  stored [K][ldb >= N] and contracted over its rows (the forward
 *          weight codes, read transposed in the kernel);
 *     sB = the same block-scale table, [K/128][ld_sb >= N/128].
 *     N % 128 == 0.
 *  FP8_LAYOUT_DGRAD_T (M = tokens, N = d_in, K = d_out) - Dgrad from the
 *                     transposed weight codes, same result as FP8_LAYOUT_DGRAD
 *     A  = dY_q  [M][lda >= K];    sA [K/128][ld_sa >= M]     (1x128 row scales)
 *     B  = W_q^T [N][ldb >= K]     (q_t of fp8_quant_weight_128x128);
 *     sB = the forward block-scale table, [K/128][ld_sb >= N/128].
 *     N % 128 == 0.
 *  FP8_LAYOUT_WGRAD   (M = d_out, N = d_in, K = tokens)
 *     A  = dY_q^T [M][lda >= K];   sA [K/128][ld_sa >= M]     (128x1 column scales)
 *     B  = X_q^T  [N][ldb >= K];   sB [K/128][ld_sb >= N]     (128x1 column scales)
 *  FP8_LAYOUT_FPROP_TILED, FP8_LAYOUT_DGRAD_T_TILED, FP8_LAYOUT_WGRAD_TILED -
 *     FPROP, DGRAD_T and WGRAD with B in the operand-tiled layout
 *     (fp8_quant_weight_128x128_tiled's q_tiled / q_t_tiled; for WGRAD the
 *     FP8_TILE_COL_TILED or fp8_quant_act_dual_tiled codes of X); ldb must
 *     equal K and N % 128 == 0.  Bit-identical results; the B-side loads
 *     become whole contiguous lines.
 *  C: [M][ldc >= N], BF16 (round to nearest even) or FP32 (c_dtype).
 *  M == 0 is a no-op.  C must not overlap A, B or the scales.
 *  Limits (FP8_ERR_UNSUPPORTED beyond them): lda, ldb <= 2^23, each scale
 *  table (its rows x ld x 4 bytes) under 2 GiB, and fewer than 2^31 output
 *  tiles of 128 x 256 (grouped: counting one ragged tile per group).
 *  Workspace: FPROP, DGRAD_T and WGRAD run on a persistent grid of one
 *  workgroup per CU.  When the output tiles leave that grid's last round at
 *  most half full, the leftover tiles are cut along K and their FP32 partial
 *  sums added in a fixed order (the result is deterministic and within the
 *  same tolerance; it can differ from the whole-tile sum in the last bits).
 *  The partial sums live in a workspace the library allocates on the first
 *  call on `stream` (128 KB per CU plus 4 bytes per CU, kept until the
 *  process ends, one per stream and device); without one - the stream is
 *  being captured into a graph, or the allocation fails - whole tiles run.
 */
fp8_status fp8_block_gemm(fp8_gemm_layout layout, int64_t M, int64_t N, int64_t K,
                          const uint8_t* A, int64_t lda, const float* sA, int64_t ld_sa,
                          const uint8_t* B, int64_t ldb, const float* sB, int64_t ld_sb,
                          void* C, fp8_out_dtype c_dtype, int64_t ldc, void* stream);

/*
 * fp8_block_gemm_noalloc - fp8_block_gemm for callers that cannot allocate
 * (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc): the same arguments, kernels and results, with the split
 * workspace in a static device array of the library instead of an
 * allocation.  The call allocates nothing, on the device or the host.
 *  The array holds 256 pieces (one per CU): 32 MiB + 1 KiB on every GPU the
 *  library runs on, kept until the process ends.  Devices with more than
 *  256 CUs are refused (FP8_ERR_UNSUPPORTED).
 *  All calls on one GPU share the array: calls that overlap in time on one
 *  GPU (different streams, not ordered) race and give wrong results; calls
 *  on one stream are ordered and safe.  The array keeps the last call's
 *  partial sums; its counters return to zero after every launch and are
 *  cleared once per device by a kernel on `stream` at the first call.
 *  Errors: as fp8_block_gemm, plus FP8_ERR_UNSUPPORTED above.
 */
fp8_status fp8_block_gemm_noalloc(fp8_gemm_layout layout, int64_t M, int64_t N, int64_t K,
                                  const uint8_t* A, int64_t lda, const float* sA, int64_t ld_sa,
                                  const uint8_t* B, int64_t ldb, const float* sB, int64_t ld_sb,
                                  void* C, fp8_out_dtype c_dtype, int64_t ldc, void* stream);

/*
 * fp8_block_gemm_fused_quant - FPROP with the 1x128 quantization of X fused
 * into the GEMM ("Online Quantization During Training", section 5: fusing
 * the scaling with its neighbours decides whether online scaling is
 * affordable; "FP8 Mixed Precision: DeepSeek-V3 Training Architecture",
 * section 3):  Y = fp8_block_gemm(FPROP, quant_1x128(X), W_q)  in one launch,
 * the codes formed on chip by every output tile's workgroup.
 *  x      BF16 X [M][ldx >= K], 16-byte aligned, ldx % 8 == 0, ldx <= 2^22.
 *  W      W_q [N][ldw >= K] (row-major codes), sW [N/128][ld_sw >= K/128].
 *  C      [M][ldc >= N], BF16 or FP32; bit-identical to fp8_quant_act_1x128
 *         (ROW, online scales) followed by fp8_block_gemm (FPROP).
 *  q_out, s_out  optional (both NULL or both set): the codes [M][ldq >= K]
 *         and scales [K/128][ld_s >= M] the kernel formed, equal to
 *         fp8_quant_act_1x128's outputs.
 *  N % 128 == 0, K % 128 == 0.  M == 0 is a no-op.  C must not overlap the
 *  inputs; q_out and s_out must not overlap C, X or each other.
 */
fp8_status fp8_block_gemm_fused_quant(int64_t M, int64_t N, int64_t K, const void* x, int64_t ldx,
                                     const uint8_t* W, int64_t ldw, const float* sW, int64_t ld_sw,
                                     void* C, fp8_out_dtype c_dtype, int64_t ldc, uint8_t* q_out,
                                     int64_t ldq, float* s_out, int64_t ld_s, void* stream);

/*
 * fp8_block_gemm_grouped - one launch of per-expert FPROP GEMMs over row
 * slices (one GPU's share of a mixture-of-experts FFN layer):
 *     for g in [0, groups): rows offsets[g] .. offsets[g+1]-1 of A and C use
 *     expert weights B_g.
 *  offsets_dev  DEVICE int32 [groups + 1], non-decreasing prefix sums with
 *               offsets[0] == 0 and offsets[groups] == total_M.  It is not
 *               read on the host.  Empty groups are allowed.  The kernel
 *               clamps what it reads so that no access leaves rows
 *               [0, total_M) of A, sA and C whatever the array holds: group
 *               g covers rows [lo, hi) with lo = min(max(offsets[g], 0),
 *               total_M) and hi = min(max(offsets[g+1], lo), total_M), so a
 *               decreasing pair gives an empty group.  For an array that
 *               breaks the contract the values of C are unspecified
 *               (clamped groups may overlap), but C is never written
 *               outside those rows.
 *  A   X_q [total_M][lda >= K];  sA [K/128][ld_sa >= total_M]
 *  B   W_q [groups][N][ldb >= K] (group g at B + g * N * ldb)
 *  sB  [groups][N/128][K/128] contiguous
 *  C   [total_M][ldc >= N], BF16 or FP32.   N % 128 == 0, K % 128 == 0.
 *  The tiles are counted on the device from the offsets; the split of
 *  leftover tiles and its per-stream workspace are as for fp8_block_gemm.
 *  Limits as for fp8_block_gemm.
 */
fp8_status fp8_block_gemm_grouped(int32_t groups, const int32_t* offsets_dev, int64_t total_M,
                                  int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                  const float* sA, int64_t ld_sa, const uint8_t* B, int64_t ldb,
                                  const float* sB, void* C, fp8_out_dtype c_dtype, int64_t ldc,
                                  void* stream);

/*
 * fp8_block_gemm_grouped_tiled - fp8_block_gemm_grouped with each expert's
 * B_g in the operand-tiled layout (N * K bytes per expert, expert g at
 * B + g * N * K); bit-identical results.
 */
fp8_status fp8_block_gemm_grouped_tiled(int32_t groups, const int32_t* offsets_dev, int64_t total_M,
                                        int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                        const float* sA, int64_t ld_sa, const uint8_t* B,
                                        const float* sB, void* C, fp8_out_dtype c_dtype,
                                        int64_t ldc, void* stream);

/*
 * fp8_amax_history_update - per-tile state of the exponential amax-history
 * (delayed) scale policy ("Online Quantization During Training", section 4
 * and worked example; "Introduction to LLM Quantization", section 5):
 *     init != 0:  h = amax
 *     otherwise:  h = fl32(fl32(decay * h) + fl32(fl32(1 - decay) * amax))
 *     scales_out (optional) = max(fl32(h / 448), fl32(1e-12)), NaN -> 0x7FC00000
 *  hist, amax, scales_out: FP32 device arrays of n elements.
 */
fp8_status fp8_amax_history_update(float* hist, const float* amax, int64_t n, float decay,
                                   int init, float* scales_out, void* stream);

/*
 * fp8_cast_e4m3 - the saturating round-to-nearest-even FP32 -> E4M3 cast the
 * quantizers use, exposed on its own (n elements, any alignment).
 */
fp8_status fp8_cast_e4m3(const float* x, int64_t n, uint8_t* q, void* stream);

/*
 * fp8_quant_act_tiles - the online rule with a chosen tile size and
 * percentile clipping ("Fine-Grained FP8 Quantization in DeepSeek", section
 * 2 and its study lab: error against tile size, scale metadata cost;
 * "Online Quantization During Training", section 4: percentile clipping).
 *  x       BF16 [rows][ldx >= cols]; cols % tile == 0.
 *  tile    T in {32, 64, 128, 256, 512, 1024}: tiles of 1 x T contiguous
 *          values of a row.
 *  rank    1..8: the clip value c is the rank-th largest |x| of the tile
 *          (1 = the max: with T = 128 the output equals fp8_quant_act_1x128
 *          ROW); s = max(fl32(c / 448), fl32(1e-12)); the rank - 1 values
 *          above c saturate.  A tile holding NaN: scale NaN, codes NaN.
 *  q       [rows][ldq >= cols] codes;  scales [cols/T][ld_s >= rows] FP32.
 *  sat_count  optional device uint32, incremented by the number of values
 *          with |fl32(x / s)| > 464 (Inf included, NaN not); caller zeroes it.
 *  Other tile or rank values: FP8_ERR_UNSUPPORTED.
 */
fp8_status fp8_quant_act_tiles(const void* x, int64_t rows, int64_t cols, int64_t ldx, int32_t tile,
                               int32_t rank, uint8_t* q, int64_t ldq, float* scales, int64_t ld_s,
                               uint32_t* sat_count, void* stream);

/*
 * fp8_gemm_promotion - accumulation-precision study: C = A . B^T over E4M3
 * codes with unit scales, FP32 out, with a chosen promotion interval
 * ("Introduction to LLM Quantization", section 3: tensor cores keep FP8 sums
 * with limited precision, so partial sums are promoted to FP32 at a fixed
 * interval; "FP8 Mixed Precision: DeepSeek-V3 Training Architecture",
 * section 3).
 *  A  [M][lda >= K] codes, B [N][ldb >= K] codes (both K-contiguous);
 *     K % 128 == 0, lda % 16 == 0, ldb % 16 == 0.
 *  promote_k  a multiple of 128: the matrix unit's accumulator is carried
 *             over promote_k / 128 consecutive 128-wide K blocks, then added
 *             to an FP32 running sum (128 = the method, bit-identical to
 *             fp8_block_gemm FPROP with unit scales and FP32 output;
 *             >= K = a single accumulator chain).  32 or 64: each 128-wide
 *             block's partial is formed per 32- or 64-wide sub-block and each
 *             is added to the running sum.  Other values: FP8_ERR_UNSUPPORTED.
 *  C  FP32 [M][ldc >= N]; must not overlap A or B.
 *  A reference kernel (one wave per 16x16 tile), not tuned for speed.
 */
fp8_status fp8_gemm_promotion(const uint8_t* A, int64_t M, int64_t K, int64_t lda, const uint8_t* B,
                              int64_t N, int64_t ldb, int64_t promote_k, float* C, int64_t ldc,
                              void* stream);

/*
 * FP8 token payloads - one self-contained message per token for activations
 * kept for the backward pass and for the tokens sent to experts in the MoE
 * all-to-all ("FP8 Mixed Precision: DeepSeek-V3 Training Architecture",
 * section 4: cached activations and dispatched tokens in FP8, and its section
 * on the MoE all-to-all: each dispatched token is one hidden vector).
 *
 * Message layout for H channels (H % 128 == 0), H + H/32 bytes:
 *   bytes [0, H)           E4M3 codes of the token's 1x128 tiles (the online
 *                          rule above, identical to fp8_quant_act_1x128 ROW)
 *   bytes [H, H + H/32)    the H/128 FP32 tile scales, little-endian, in tile order
 * Messages sit at `stride` bytes (stride >= H + H/32, stride % 16 == 0);
 * bytes past a message are not written.  7168 channels: 7392 bytes, 33/64 of
 * the BF16 row.
 */

/*
 * fp8_pack_tokens - quantize tokens into messages.
 *  x         BF16 [x_rows][ldx >= H]
 *  src_rows  optional int32 [T] device array: message t carries row
 *            src_rows[t] (the dispatch order; rows may repeat).  NULL: row t
 *            (then T <= x_rows).  A src_rows entry outside [0, x_rows) gives a
 *            message of NaN codes (0x7F) and NaN scales (0x7FC00000).
 *  msg       [T][stride] bytes; must not overlap x or src_rows.
 */
fp8_status fp8_pack_tokens(const void* x, int64_t x_rows, int64_t H, int64_t ldx,
                           const int32_t* src_rows, int64_t T, uint8_t* msg, int64_t stride,
                           void* stream);

/*
 * fp8_unpack_tokens - messages into the GEMM operand layout of
 * fp8_quant_act_1x128 ROW: codes q [T][ldq >= H] and MN-major scales
 * [H/128][ld_s >= T] (byte copies: bit-exact).  Outputs must not overlap msg
 * or each other.
 */
fp8_status fp8_unpack_tokens(const uint8_t* msg, int64_t T, int64_t H, int64_t stride, uint8_t* q,
                             int64_t ldq, float* scales, int64_t ld_s, void* stream);

/*
 * fp8_dequant_tokens - restore BF16 from messages: y [T][ldy >= H] with
 * y = decode(q) * s rounded once to BF16 (nearest, ties to even) from the
 * exact product; NaN codes or scales give 0x7FC0, 0 * Inf gives 0x7FC0.
 * y must not overlap msg.
 */
fp8_status fp8_dequant_tokens(const uint8_t* msg, int64_t T, int64_t H, int64_t stride, void* y,
                              int64_t ldy, void* stream);

/* Static string naming a status; never NULL. */
const char* fp8_status_string(fp8_status s);

/* FP8BS_ABI_VERSION of the built library. */
int fp8_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
