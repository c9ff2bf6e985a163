/*
 * bq_debug.h -- test and measurement hooks of libbq.  bq_debug_nearest_codes makes no HIP call
 * and works without a GPU; bq_debug_time_next_kernel only arms events that a later call
 * fills.
 */
#ifndef BQ_DEBUG_H
#define BQ_DEBUG_H

#include "bq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Replays on the host, for `count` binary32 values y[i], the nearest-code search exactly as
 * the quantize kernels perform it: the decision thresholds T_k (smallest binary32 above each
 * midpoint of adjacent entries), the bucket function and LUT chosen for this table, and the
 * per-element compares; non-finite y give the zero code.  This defines the same result as
 * the "nearest" rule of bq.h for |y| <= 1 and lets the table preparation be tested without a
 * GPU.
 *   table     [host] as for bq_quantize_blockwise (validated the same way).
 *   y, codes  [host] count inputs and count outputs.
 *   mode      [host] out (may be NULL): 0 uniform buckets, 1 logarithmic buckets,
 *             2 binary search.
 *   compares  [host] out (may be NULL): threshold compares per element in bucket modes.
 * Returns BQ_OK, BQ_ERR_NULL or BQ_ERR_TABLE. */
bq_status bq_debug_nearest_codes(const bq_code_table* table, const float* y, int64_t count,
                                 int32_t* codes, int32_t* mode, int32_t* compares);

/* Measurement hook: the next kernel the library launches on the calling thread goes through
 * hipExtLaunchKernel with these events; then the hook forgets both.  The next call's first
 * kernel is the one armed: the data kernel of a nested quantize (bq_quantize_nested or
 * bq_quantize_nested_noalloc), or the only kernel of the other calls.  `stop` (if not NULL) is
 * bound to that kernel and takes its end time, adding nothing to the kernel.  `start` (if not
 * NULL) becomes a marker enqueued just before the kernel: on MI355X with ROCm 7.2 its
 * timestamp leads the kernel's own start by a near-constant 4.4-5.4 us, so
 * hipEventElapsedTime(start, stop) over one launch overstates it by that lead (two markers
 * recorded back to back span about the same time, 4.1 us, and measure it).  Any armed
 * launch also leaves the GPU idle for about 4.5 us after the kernel.  The events
 * are the caller's (created with timing enabled) and must stay valid until the work completes.
 * A call that fails validation launches nothing and leaves the hook armed.  Two NULLs disarm
 * it.  Returns BQ_OK. */
bq_status bq_debug_time_next_kernel(hipEvent_t start, hipEvent_t stop);

#ifdef __cplusplus
}
#endif

#endif /* BQ_DEBUG_H */
