/*
 * bq.h -- blockwise absmax quantization and dequantization for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbq.so.  Every entry point validates its arguments on the host, then enqueues
 * its kernels on the caller's HIP stream and returns without waiting.  The library never
 * allocates or frees device memory, never copies between host and device, and never
 * synchronizes, so every call can be captured in a HIP graph.
 *
 * Conventions shared by all entry points
 *   - Device pointers (marked [device]) must be device memory of the current device, and
 *     data arrays must be 16-byte aligned (fp32 statistic arrays: 4-byte aligned).  The
 *     caller owns every buffer and keeps it alive until the enqueued work completes.
 *   - Host pointers (marked [host]) are read during the call only.
 *   - `stream` is the HIP stream to enqueue on; 0 is the legacy null stream.  This follows
 *     "Respect the current CUDA stream in blockwise quantization" (bitsandbytes PR 2052),
 *     Summary: quantization must run on the caller's current stream, not stream 0.
 *   - Errors: every check happens before any HIP call; on error nothing is enqueued and no
 *     output is written.  A failed launch returns BQ_ERR_HIP.  n == 0 is valid and enqueues
 *     nothing.  Element data is never inspected on the host (that would need a sync).
 *   - Determinism: outputs are bit-identical across runs, streams and devices of this kind.
 *
 * The arithmetic (each rule is also written where it is implemented):
 *   blocks      element i belongs to block i / B of the flattened 1-D array; the last
 *               block may be partial ("full blocks, and tails", PR 2052, "Correctness and
 *               safety"); B is a power of two from 32 to 4096 (PR 2052, Summary).
 *   absmax      a_b = max |x_i| over the finite elements of block b; +0 if there are none.
 *   normalize   y_i = fl32(fl32(x_i * s) * fl32(1 / fl32(a_b * s))), s = 2^64 if
 *               a_b < 2^-64, s = 2^-64 if a_b > 2^64, else 1 (|y_i| <= 1).
 *   nearest     q_i = the smallest index k minimizing |y_i - c_k| exactly (equal distances
 *               resolve to the lowest index, as in "[OMNIML-5899] Add CUDA kernels for IQ
 *               packing", review item "Search equivalence").  Non-finite x_i and every
 *               element of a block with a_b = 0 take z = the nearest code to 0.0.
 *   packing     16-entry table: two codes per byte, the first element of each pair in the
 *               high nibble, ceil(n/2) bytes, a zero pad nibble for odd n (33 values fill
 *               17 bytes, as in onnxruntime/mobius PR 794, finding F3).  256-entry table:
 *               one byte per element.
 *   dequantize  out_i = RN(fl32(c[q_i] * a_b)): one binary32 multiply, then one
 *               round-to-nearest-even to the output type (overflow to infinity, signed zeros
 *               and subnormals kept, NaN to a quiet NaN of the same sign).
 */
#ifndef BQ_H
#define BQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the unquantized side. */
typedef enum { BQ_F32 = 0, BQ_F16 = 1, BQ_BF16 = 2 } bq_dtype;

typedef enum {
  BQ_OK = 0,
  BQ_ERR_NULL = 1,      /* a required pointer is NULL */
  BQ_ERR_DTYPE = 2,     /* dtype is not a bq_dtype */
  BQ_ERR_SIZE = 3,      /* n < 0, more than INT32_MAX blocks, n not a whole number of rows, or a
                           launch of more than 2^32 - 1 threads, refused before any work is
                           enqueued (quantize and 4-bit dequantize from 2^37 elements, 8-bit
                           dequantize from 2^36) */
  BQ_ERR_BLOCKSIZE = 4, /* blocksize not a power of two in [32, 4096] */
  BQ_ERR_TABLE = 5,     /* code table: size, order, range or spacing (see bq_code_table) */
  BQ_ERR_ALIGNMENT = 6, /* a device pointer is not aligned as required */
  BQ_ERR_FORMAT = 7,    /* unknown bq_q32_format, or row_len not a multiple of 32 (of 256 for
                           the IQ2_XS- and IQ1_S-style calls) */
  BQ_ERR_WORKSPACE = 8, /* nested workspace missing or smaller than bq_nested_workspace_bytes */
  BQ_ERR_HIP = 9        /* the HIP runtime rejected a launch */
} bq_status;

/* A code table in host memory: `size` (16 or 256) binary32 entries, strictly ascending,
 * each finite and within [-1, 1], every nonzero entry of magnitude >= 2^-20 (so that sums
 * of two entries are exact in binary64); -0.0 is read as +0.0.  16 entries select 4-bit
 * codes (packed two per byte), 256 entries 8-bit codes.  The table is read during the call
 * and passed to the kernels by value; nothing is uploaded. */
typedef struct {
  const float* entries; /* [host] */
  int32_t size;
} bq_code_table;

/* Blockwise quantization (General8 / FP4 / NF4 family of "Respect the current CUDA stream
 * in blockwise quantization", bitsandbytes PR 2052, Summary and "Correctness and safety").
 *   in         [device] n elements of `dtype`, read only.
 *   absmax     [device] out: ceil(n / blocksize) binary32 block maxima.
 *   packed     [device] out: ceil(n / 2) bytes (16-entry table) or n bytes (256 entries). */
bq_status bq_quantize_blockwise(const void* in, bq_dtype dtype, int64_t n, int32_t blocksize,
                                const bq_code_table* code_table, float* absmax, uint8_t* packed,
                                hipStream_t stream);

/* Blockwise dequantization, the inverse of bq_quantize_blockwise: one binary32 multiply of
 * the code's table entry by the block absmax, rounded once to `dtype`.
 *   out        [device] out: n elements of `dtype`.
 *   absmax     [device] ceil(n / blocksize) binary32 values (any values; NaN propagates).
 *   packed     [device] codes laid out as bq_quantize_blockwise writes them. */
bq_status bq_dequantize_blockwise(void* out, bq_dtype dtype, int64_t n, int32_t blocksize,
                                  const bq_code_table* code_table, const float* absmax,
                                  const uint8_t* packed, hipStream_t stream);

/* Second-level statistics of nested quantization (nested General8 and compressed-statistics
 * NF4 of PR 2052, "Reproduced failure").  The block absmax values a_b are replaced by:
 *   mean     = RN32(S / nb), S the binary64 pairwise sum of a_0 .. a_{nb-1} zero-padded to a
 *              power-of-two length (sum of a range = sum of its left half + sum of its right);
 *   d_b      = fl32(a_b - mean), quantized with the 256-entry `table` in groups of
 *              `blocksize2` blocks by the same absmax / normalize / nearest rules;
 *   rebuilt  a'_b = fl32(fl32(c2[q2_b] * absmax2_g) + mean), used by the nested dequantize. */
typedef struct {
  uint8_t* qabsmax;            /* [device] nb codes q2_b (nb = ceil(n / blocksize)), 16-byte aligned */
  float* absmax2;              /* [device] ceil(nb / blocksize2) binary32 group maxima */
  float* mean;                 /* [device] 1 binary32 value */
  const bq_code_table* table;  /* [host] 256-entry statistics table */
  int32_t blocksize2;          /* blocks per statistics group: power of two in [32, 4096] */
  void* workspace;             /* [device] scratch, 256-byte aligned; quantize only */
  size_t workspace_bytes;
} bq_nested_stats;

/* Bytes of device workspace bq_quantize_nested needs (0 for n <= 0), for any dtype.  After the
 * call's stream work completes, the workspace starts with the nb = ceil(n / blocksize) block
 * maxima a_b: nb binary32 values for BQ_F32 input; for BQ_F16 / BQ_BF16 input, nb 16-bit
 * values of that type (the maximum of |x| over values of a format is itself a value of the
 * format, so they are exact). */
size_t bq_nested_workspace_bytes(int64_t n, int32_t blocksize, int32_t blocksize2);

/* Blockwise quantization with nested statistics: packed data codes as bq_quantize_blockwise,
 * and the statistics of bq_nested_stats written to stats->qabsmax, ->absmax2 and ->mean.
 * Enqueues up to four kernels on `stream`: the data pass, the partial-sum runs (inputs of more
 * than 2^20 elements), the mean (more than 2^31 elements), then the statistics. */
bq_status bq_quantize_nested(const void* in, bq_dtype dtype, int64_t n, int32_t blocksize,
                             const bq_code_table* code_table, bq_nested_stats* stats,
                             uint8_t* packed, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): bq_quantize_nested with the library's own scratch
 * memory in place of the caller's workspace.  stats->workspace and stats->workspace_bytes are
 * ignored; everything else, the outputs and the errors are those of bq_quantize_nested.
 * The scratch is a fixed 36 MiB array per GPU (37,748,736 bytes, held by every GPU the library
 * runs on until the process ends), enough for any input whose bq_nested_workspace_bytes is at
 * most that size, e.g. 2^29 elements at block size 64; a larger input returns
 * BQ_ERR_WORKSPACE before anything is enqueued.  The call allocates nothing.  All calls on one
 * GPU share its scratch, which keeps the last call's contents: calls that overlap on one GPU
 * (two streams or host threads without ordering between them) race and give wrong results. */
bq_status bq_quantize_nested_noalloc(const void* in, bq_dtype dtype, int64_t n, int32_t blocksize,
                                     const bq_code_table* code_table, bq_nested_stats* stats,
                                     uint8_t* packed, hipStream_t stream);

/* Dequantization from nested statistics: rebuilds each a'_b from (q2_b, absmax2_g, mean) and
 * dequantizes with it, in one kernel.  stats->workspace is not used. */
bq_status bq_dequantize_nested(void* out, bq_dtype dtype, int64_t n, int32_t blocksize,
                               const bq_code_table* code_table, const bq_nested_stats* stats,
                               const uint8_t* packed, hipStream_t stream);

/* GGUF-style 32-element blocks (the Q4_0 / Q8_0 shapes of "Cache device-side constants in
 * dequant kernels", ComfyUI-GGUF PR 472, "Verification" table):
 *   BQ_Q32_Q4: 18 bytes = binary16 scale d (little-endian) + 16 bytes; element j < 16 is the
 *              low nibble of byte j, element 16 + j its high nibble (the low-before-high
 *              nibble order of that page's "Problem" section); value (q - 8) * d.
 *   BQ_Q32_Q8: 34 bytes = binary16 d + 32 int8; value q * d.
 * The binary32 product is exact; it is rounded once to `dtype`. */
typedef enum { BQ_Q32_Q4 = 0, BQ_Q32_Q8 = 1 } bq_q32_format;

/* Dequantizes n / 32 consecutive blocks (row-major rows of row_len elements; row_len a
 * multiple of 32 dividing n, so no block straddles a row: the per-row alignment check of
 * "[OMNIML-5899] Add CUDA kernels for IQ packing").
 *   blocks  [device] (n / 32) * 18 or * 34 bytes, 2-byte aligned (the records themselves are;
 *           a slice starting at any block is accepted; 16-byte aligned arrays are read faster).
 *   out     [device] out: n elements of `dtype`. */
bq_status bq_dequant_q32(const void* blocks, bq_dtype dtype, int64_t n, int32_t row_len,
                         bq_q32_format format, void* out, hipStream_t stream);

/* Fused dequantize + linear for small batches (decoding): y = x . deq(W)^T, with the
 * dequantized weights formed in registers and never written out (weights used without
 * expanding the full tensor, as in the mixed-input GEMMs of "stable-diffusion.cpp PR 2278",
 * Summary; here for the blockwise codes of bq_quantize_blockwise).
 *   x          [device] M x K row-major activations of `dtype`, 16-byte aligned.
 *   M, K, N    1 <= M <= 4; K > 0 and a multiple of 16; 0 <= N <= 67,108,860 (a launch holds
 *              at most 2^32 - 1 threads; N = 0: nothing enqueued).
 *   blocksize, code_table
 *              the block size and table W was quantized with.
 *   absmax     [device] ceil(N*K / blocksize) binary32 block maxima of W.
 *   packed     [device] W's codes, 16-byte aligned, as bq_quantize_blockwise writes them for
 *              the N*K-element weight tensor stored row-major (element (n, k) of W is flat
 *              element n*K + k; blocks run over the flat index).
 *   y          [device] out: M x N row-major binary32.
 * y[m][n] approximates sum_k x[m][k] * w[n][k], w = fl32(c[q] * a) the binary32 dequantized
 * weight (never rounded to 16 bits), accumulated in binary32 in an unspecified order: its
 * error is at most (K/1024 + 64) * 2^-24 * sum_k |x[m][k] w[n][k]|.
 * Errors: BQ_ERR_SIZE for M outside [1, 4], K not a positive multiple of 16, N outside
 * [0, 67108860], or more than INT32_MAX blocks; otherwise as bq_dequantize_blockwise. */
bq_status bq_linear_blockwise(const void* x, bq_dtype dtype, int64_t M, int64_t K, int64_t N, int32_t blocksize,
                              const bq_code_table* code_table, const float* absmax, const uint8_t* packed,
                              float* y, hipStream_t stream);

/* Fused dequantize + GEMM on the matrix cores, for batches of rows (the 16-bit-activation,
 * 4-bit-weight GEMM named in "stable-diffusion.cpp PR 2278", Summary, here for the blockwise
 * codes of bq_quantize_blockwise): y = x . W16^T, where W16 is exactly the 16-bit tensor
 * bq_dequantize_blockwise writes for W with this `dtype`, w16 = RN16(fl32(c[q] * a)), formed
 * in registers and never written out.
 *   x          [device] M x K row-major activations, BQ_BF16 or BQ_F16, 16-byte aligned.
 *   M, K, N    M >= 1 (at most 4,194,240); K > 0 and a multiple of 64; 0 <= N <= 536,870,848
 *              (a launch holds at most 2^32 - 1 threads; N = 0: nothing enqueued).
 *   blocksize, code_table, absmax, packed
 *              W, as for bq_linear_blockwise (packed 16-byte aligned).
 *   y          [device] out: M x N row-major binary32.
 * Each product x[m][k] * w16[n][k] is exact in binary32; the products are accumulated in
 * binary32 in an unspecified order, so y[m][n] lies within (K + 64) * 2^-24 * sum_k
 * |x[m][k] w16[n][k]| of the exact sum (products below the binary32 normal range may be
 * flushed to zero by the matrix cores).  The result is the same on every call on one device.
 * Errors: BQ_ERR_DTYPE for BQ_F32; BQ_ERR_SIZE for M outside [1, 4194240], K not a positive
 * multiple of 64, N outside [0, 536870848], or more than INT32_MAX blocks; otherwise as
 * bq_dequantize_blockwise. */
bq_status bq_gemm_blockwise(const void* x, bq_dtype dtype, int64_t M, int64_t K, int64_t N, int32_t blocksize,
                            const bq_code_table* code_table, const float* absmax, const uint8_t* packed,
                            float* y, hipStream_t stream);

/* IQ2_XS-style search encoding ("[OMNIML-5899] Add CUDA kernels for IQ packing", Model-
 * Optimizer PR 2448: the Summary's caller-computed fp16 superblock scales, the review items
 * "Wire format", "Scale anchors", "Even-parity sign field" and "Search equivalence", and the
 * round-3 "IQ2_XS grouping" item).  A superblock is 256 consecutive elements, stored in 74
 * bytes:
 *   bytes 0-1   the caller's binary16 scale d (little-endian);
 *   bytes 2-65  32 little-endian 16-bit words, one per 8-element vector v: bits 0-8 the grid
 *               entry e, bits 9-15 the signs of the vector's elements 0-6 (bit set =
 *               negative); element 7's sign is the parity of those seven bits, so every
 *               vector holds an even number of negative elements;
 *   bytes 66-73 byte i = ls[2i] | ls[2i+1] << 4, the 4-bit local scale of each 16-element
 *               group g (vectors 2g and 2g+1).
 * Element j of vector v decodes to d * (2 * ls + 1) / 8 * grid[e][j], negated if its sign is
 * set (exact in binary32, then rounded once to the output type).
 * The grid is the caller's: 512 entries of 8 magnitude bytes (entry e, element j at byte
 * 8e + j), for the IQ2_XS format those of the GGML grid (bytes 0x08, 0x19, 0x2b).
 *
 * The search, per superblock with a valid d (binary32 throughout, fused multiply-adds where
 * written fma, every other operation rounded once):
 *   a_j = |x_j| (a NaN or infinite element reads as +0; -0 is not negative);
 *   xn = fma-chain sum of a_j^2 and dot_e = fma-chain sum of a_j * q_j (j = 0..7, from +0);
 *   with an odd count of negative elements, dot_e = fma(-2, w_e, dot_e), w_e the least
 *   fl(a_j * q_j), and the first element reaching w_e has its sign flipped;
 *   s = d * (2 * ls + 1) / 8; error(e, s) = max(fma(s*s, qn_e, fma(-2s, dot_e, xn)), 0),
 *   qn_e = sum of q_j^2;
 *   each group takes the ls whose fl(E(v0) + E(v1)) is least (E(v) = least error of vector v
 *   over the grid; equal sums: the lower ls), then each vector the entry of least error at
 *   that ls (equal errors: the lower entry).
 * Scales: d = +0 or -0 gives an all-zero superblock.  A NaN, infinite or negative d is
 * rejected: the superblock is written as zeros and *rejected is incremented (atomically, on
 * the device: the caller sets it beforehand and reads it after the stream work completes).
 *   in        [device] n elements of `dtype`, 16-byte aligned.
 *   n, row_len  row_len a positive multiple of 256 dividing n (n = 0: nothing enqueued), so no
 *             superblock straddles a row (the per-row check of that page's round-3 review).
 *   grid      [device] 4096 bytes, 16-byte aligned.
 *   scales    [device] n / 256 binary16 bit patterns, 2-byte aligned.
 *   blocks    [device] out: (n / 256) * 74 bytes, 2-byte aligned.
 *   rejected  [device] one uint32 counter, 4-byte aligned.
 * Errors: BQ_ERR_DTYPE, BQ_ERR_FORMAT (row_len), BQ_ERR_SIZE (n negative or not a multiple of
 * row_len, more than INT32_MAX superblocks), BQ_ERR_NULL, BQ_ERR_ALIGNMENT, BQ_ERR_HIP. */
bq_status bq_iq2xs_quantize(const void* in, bq_dtype dtype, int64_t n, int64_t row_len, const uint8_t* grid,
                            const uint16_t* scales, uint8_t* blocks, uint32_t* rejected, hipStream_t stream);

/* Decodes n / 256 superblocks laid out as bq_iq2xs_quantize writes them (any bytes: d is read
 * as binary16 whatever it holds) to n elements of `dtype`.
 *   blocks    [device] (n / 256) * 74 bytes, 2-byte aligned.
 *   grid      [device] 4096 bytes, 8-byte aligned.
 *   out       [device] out: n elements of `dtype`, 16-byte aligned.
 * Errors: as bq_iq2xs_quantize. */
bq_status bq_iq2xs_dequantize(const uint8_t* blocks, const uint8_t* grid, int64_t n, int64_t row_len,
                              bq_dtype dtype, void* out, hipStream_t stream);

/* IQ1_S-style encoding ("[OMNIML-5899] Add CUDA kernels for IQ packing", Model-Optimizer PR
 * 2448: "Provenance" (16.875 = 15 x (1 + 1/8), the 0.61 scale predictor, the 0.125 delta), the
 * review items "Wire format", "Scale anchors" and "Search equivalence", the round-3 item on
 * the shifted objective).  A superblock is 256 consecutive elements, stored in 50 bytes:
 *   bytes 0-1   binary16 scale d (little-endian);
 *   bytes 2-33  byte v = the low 8 bits of vector v's 11-bit grid entry (vector v = elements
 *               8v .. 8v+7);
 *   bytes 34-49 8 little-endian 16-bit words, one per 32-element sub-block b (vectors
 *               4b .. 4b+3): bits 3l..3l+2 the high 3 bits of vector 4b+l's entry, bits 12-14
 *               the local scale ls, bit 15 the delta sign (set: delta = -1/8, else +1/8).
 * Element j of vector v decodes to fl32(d * (2 ls + 1) * (g_j + delta)), g the grid's signed
 * byte (exact for the ternary IQ1_S grid), rounded once to the output type.
 * The grid is the caller's: 2048 entries of 8 signed bytes (entry e, element j at byte 8e + j),
 * for the IQ1_S format those of the GGML ternary grid (-1, 0, +1).
 *
 * The encoder, per superblock (binary32 throughout, fused multiply-adds where written fma):
 *   x_j = the element, a NaN or infinite element read as +0;
 *   d = RN16(fl32(fl32(amax / 16.875) * 0.61)), amax = max |x_j| over the superblock,
 *   saturated to the largest finite binary16; d = 0 gives an all-zero superblock;
 *   per vector: xn, dot_e and xsum are fma chains of x_j^2, x_j * g_j and x_j * 1 (j = 0..7,
 *   from +0); for a choice c = ls + 8 * sign, dl = d * (2 ls + 1), delta = +-1/8:
 *   error(e, c) = max(fma(dl*dl, sn, fma(-2 dl, fma(delta, xsum, dot_e), xn)), 0),
 *   sn = qn_e + 2 delta qs_e + 8 delta^2 (qn, qs = sum of g^2 and of g);
 *   each sub-block takes the choice whose summed error over its four vectors (in vector
 *   order) is least (equal sums: the lower c), then each vector the entry of least error at
 *   that choice (equal errors: the lower entry).
 *   in        [device] n elements of `dtype`, 16-byte aligned.
 *   n, row_len  row_len a positive multiple of 256 dividing n (n = 0: nothing enqueued).
 *   grid      [device] 16384 bytes, 16-byte aligned.
 *   blocks    [device] out: (n / 256) * 50 bytes, 2-byte aligned.
 * Errors: BQ_ERR_DTYPE, BQ_ERR_FORMAT (row_len), BQ_ERR_SIZE (n negative or not a multiple of
 * row_len, more than INT32_MAX superblocks), BQ_ERR_NULL, BQ_ERR_ALIGNMENT, BQ_ERR_HIP. */
bq_status bq_iq1s_quantize(const void* in, bq_dtype dtype, int64_t n, int64_t row_len, const int8_t* grid,
                           uint8_t* blocks, hipStream_t stream);

/* Decodes n / 256 superblocks laid out as bq_iq1s_quantize writes them (any bytes) to n
 * elements of `dtype`.
 *   blocks    [device] (n / 256) * 50 bytes, 2-byte aligned.
 *   grid      [device] 16384 bytes, 8-byte aligned.
 *   out       [device] out: n elements of `dtype`, 16-byte aligned.
 * Errors: as bq_iq1s_quantize. */
bq_status bq_iq1s_dequantize(const uint8_t* blocks, const int8_t* grid, int64_t n, int64_t row_len,
                             bq_dtype dtype, void* out, hipStream_t stream);

/* The hipError_t (as int) of the most recent launch that failed on the calling thread with
 * BQ_ERR_HIP, or 0 if none has. */
int bq_last_hip_error(void);

/* Static description of a status code (never NULL). */
const char* bq_status_string(bq_status status);

#ifdef __cplusplus
}
#endif

#endif /* BQ_H */
