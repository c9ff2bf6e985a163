/*
 * bq_debug.h -- test hooks of libbq (host only; no HIP call, usable without a GPU).
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

#ifdef __cplusplus
}
#endif

#endif /* BQ_DEBUG_H */
