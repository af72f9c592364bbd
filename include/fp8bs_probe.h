/*
 * fp8bs_probe.h - measurement and verification aids exported by libfp8bs.so.
 *
 * Nothing here is a step of the quantization method or of the block-scaled
 * GEMM.  These calls exist so that a roofline can be put beside the GEMMs'
 * measured rate (the matrix unit's sustained rate with no memory traffic) and
 * so that a step of the quantizers' arithmetic can be checked exhaustively.
 * The split query reports how the GEMM kernel schedules a launch.
 * They follow the conventions of fp8bs.h: caller-owned device buffers,
 * host-side validation before any launch, asynchronous on `stream`, and an
 * fp8_status result.
 */
#ifndef FP8BS_PROBE_H
#define FP8BS_PROBE_H

#include "fp8bs.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Instruction mix of fp8_probe_mfma. */
typedef enum {
  FP8_PROBE_MFMA_PLAIN = 0,  /* v_mfma_f32_16x16x128_f8f6f4, 8 accumulator chains
                                (the GEMMs' instruction) */
  FP8_PROBE_MFMA_SCALED = 1, /* the block-scaled encoding of the same product,
                                E8M0 scales 2^0 (a scale-load prefix per MFMA) */
  FP8_PROBE_MFMA_FOLD = 2    /* plain MFMAs with a zero accumulator, each followed
                                by the 4 FP32 FMAs folding the previous partial of
                                its chain (the GEMMs' per-K-block mix) */
} fp8_probe_mfma_mode;

/*
 * fp8_probe_mfma - each wave runs 8 independent chains of FP8 MFMAs for
 * `iters` rounds with no memory traffic, so the duration gives the rate the
 * matrix unit sustains on the given operand bytes (the clock under load
 * depends on the power the data draws) for the chosen instruction mix.
 *  workgroups  1..2^20 workgroups of 256 threads (four waves); each wave does
 *              8 * iters MFMAs of 65,536 FLOP
 *  iters       >= 1
 *  mode        an fp8_probe_mfma_mode
 *  codes       device, 4096 bytes of E4M3 codes: lane l of every wave takes
 *              operand A from bytes [32 l, 32 l + 32) and B from
 *              [2048 + 32 l, 2048 + 32 l + 32); 16-byte aligned
 *  out         device, workgroups * 256 floats: per lane, the sum of its
 *              accumulators (a checksum that keeps the work observable; the
 *              same in every mode)
 *  Errors: FP8_ERR_SHAPE (sizes or mode), FP8_ERR_NULL, FP8_ERR_ALIGN,
 *  FP8_ERR_ALIAS, FP8_ERR_DEVICE, FP8_ERR_LAUNCH.
 */
fp8_status fp8_probe_mfma(int64_t workgroups, int32_t iters, int32_t mode, const uint8_t* codes,
                          float* out, void* stream);

/*
 * fp8_probe_recip_online - r[i] = the reciprocal the quantizers use for an
 * online scale s[i] (the hardware estimate refined by one Newton step through
 * FMAs), so a test can check it against the IEEE reciprocal on every scale
 * the online rule produces.
 *  s, r   device, n floats each, 4-byte aligned, not overlapping; 0 <= n <= 2^30
 *  Errors: FP8_ERR_SHAPE, FP8_ERR_NULL, FP8_ERR_ALIGN, FP8_ERR_ALIAS,
 *  FP8_ERR_DEVICE, FP8_ERR_LAUNCH.
 */
fp8_status fp8_probe_recip_online(const float* s, float* r, int64_t n, void* stream);

/*
 * fp8_probe_gemm_split - the schedule the persistent GEMM kernel (FPROP,
 * DGRAD_T, WGRAD, grouped) takes for `tiles` output tiles of 128 x 256 with
 * K-dimension `K` when enqueued on `stream` of the current device, so that a
 * test can tell whether a launch ran the split-K tail it means to check.
 * When the tiles leave the last round of one tile per workgroup at most half
 * full, each leftover tile is cut along K into pieces run by otherwise idle
 * workgroups, the last piece to finish adding the partial tiles in piece
 * order; that needs the split workspace the library holds per stream (made by
 * the first GEMM call on the stream).
 *  tiles        >= 0
 *  K            > 0, a multiple of 128
 *  split_tiles  host: receives the number of tiles run as pieces (0: none)
 *  pieces       host: receives the pieces per split tile (1: no split)
 *  Errors: FP8_ERR_SHAPE, FP8_ERR_NULL, FP8_ERR_DEVICE.
 */
fp8_status fp8_probe_gemm_split(int64_t tiles, int64_t K, void* stream, int64_t* split_tiles, int32_t* pieces);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_PROBE_H */
