/*
 * moe_ceiling.h -- reference kernels for measuring libmoe_mi355x against what
 * the MI355X memory system gives for its access patterns
 * (libmoe_ceiling.so).
 *
 * They are not part of the MoE method's path: they move the same bytes in
 * the same patterns (the gather also sums its rows, truncating to bf16, as a
 * stand-in for the combine's arithmetic).  A benchmark times them on the same
 * GPU, on buffers of the same sizes and, for the scatter and the gather,
 * along the same handle, and reports each library kernel's rate as a fraction
 * of the matching reference: a practical ceiling (for the gather, a
 * reference) beside the 8 TB/s HBM peak.
 *
 * Conventions: device pointers on the current device, 16-byte aligned;
 * `stream` is a hipStream_t passed as void* (NULL = the null stream); every
 * call only queues one kernel (no allocation, no sync) and returns
 * MOE_CEILING_OK, MOE_CEILING_ERR_ARG (bad argument, nothing launched) or
 * MOE_CEILING_ERR_HIP (the launch failed).  Sizes past one launch (a grid
 * past 2^32 work-items) are MOE_CEILING_ERR_ARG.
 */
#ifndef MOE_CEILING_H
#define MOE_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOE_CEILING_OK = 0, MOE_CEILING_ERR_ARG = 1, MOE_CEILING_ERR_HIP = 2 };

/* Zero `bytes` (a multiple of 16) of dst: one wave per piece of piece_kib
 * KiB (1, 2 or 4) in address order, non-temporal stores.  The write-only
 * pattern of the sync-free zero tail. */
int moe_ceiling_fill(void *dst, size_t bytes, int piece_kib, void *stream);

/* Copy `bytes` (a multiple of 16) from src to dst (not overlapping): one
 * wave per piece of piece_kib KiB (1, 2 or 4) in address order, plain loads
 * and non-temporal stores.  Moves as many bytes in as out. */
int moe_ceiling_copy(const void *src, void *dst, size_t bytes, int piece_kib, void *stream);

/* Write zeros to every row [0, R) of rows ([R,H] bf16, H a positive
 * multiple of 256) that row_of_slot ([T,k] int32, as a moe_handle holds it;
 * entries outside [0, R) are skipped) names: one workgroup of four waves per
 * token, the row cut into segments of seg_kib KiB (1, 2 or 4) dealt over the
 * waves, each wave storing its segment to every row of the token's slots.
 * The dispatch's destination layout and store order, without its reads. */
int moe_ceiling_scatter(const int32_t *row_of_slot, int64_t T, int32_t k, int64_t R, int32_t H,
                        void *rows, int seg_kib, void *stream);

/* The combine's reads along a handle: for every token t < T, the rows of Y
 * ([R,H] bf16, H a positive multiple of 256) that row_of_slot ([T,k] int32,
 * 1 <= k <= 64; entries outside [0, R) skipped; a repeated row is read each
 * time it is named) names, one wave per (token, segment of seg_kib KiB: 1, 2
 * or 4), the segments of four named rows loaded (non-temporal) before any is
 * added, summed in fp32 in slot order.
 *   out   [T,H] bf16 (16-byte aligned): receives each summed segment, each
 *         element's upper 16 bits (truncated, not rounded); or NULL for a
 *         read-only gather that stores nothing...
 *   sink  ...except into this int32 device word, and only when a sum has the
 *         all-ones NaN bit pattern, which finite rows never give (it keeps
 *         the loads alive); may be NULL when out is given.
 * T = 0 launches nothing. */
int moe_ceiling_gather(const int32_t *row_of_slot, int64_t T, int32_t k, int64_t R, int32_t H,
                       const void *Y, void *out, uint32_t *sink, int seg_kib, void *stream);

/* out[j] = the XCD (accelerator complex die, 0..7 on MI355X) that workgroup
 * j of a grid of `nblocks` workgroups of 256 threads (the row kernels'
 * size) ran on, from its first wave's
 * XCC_ID hardware register.  The library's row kernels assume workgroup j
 * runs on XCD j mod 8 (the combine backward's copy and dot workgroups of one
 * token period share an XCD's L2); this checks it on the running GPU. */
int moe_ceiling_xcd_map(int32_t *out, int32_t nblocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CEILING_H */
