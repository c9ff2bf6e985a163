/*
 * bq_oracle.c -- CPU oracle for blockwise absmax quantization and dequantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, scalar definition of what the
 * GPU library computes.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the library itself never does.  It shares no code, header,
 * table or constant generator with the GPU path.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (binary32 operations round once each, round-to-nearest-even; no multiply-add is fused
 * unless written as fmaf, which only the IQ2_XS error form of that section does).
 *
 * Sources (page title, then the section or passage followed):
 *  - "Respect the current CUDA stream in blockwise quantization" (bitsandbytes PR 2052):
 *    Summary (General8 / FP4 / NF4 blockwise quantization, block sizes 32 through 4096) and
 *    "Correctness and safety" (fp16 / bf16 / fp32 inputs, full blocks and tails), and
 *    "Reproduced failure" (nested General8 quantization and compressed-statistics NF4).
 *  - "[OMNIML-5899] Add CUDA kernels for IQ packing" (Model-Optimizer PR 2448): the
 *    review's "Search equivalence" item (equal error resolves to the lowest index), the
 *    Summary's non-finite normalization, and the bit-exactness finding (separately rounded
 *    binary32 operations, never fused chains).
 *  - onnxruntime/mobius PR 794, "Confirmed findings" F3: a 4-bit row of 33 values occupies
 *    17 bytes (ceil-div packing).
 *  - "Cache device-side constants in dequant kernels" (ComfyUI-GGUF PR 472), "Problem": the
 *    shift-by-{0,4} idiom placing a 32-byte group's low nibbles before its high nibbles.
 *
 * Readings where the pages are silent (each is restated where it is used):
 *  R2  absmax is the max of |x| over finite elements; no finite element gives +0.
 *  R3  y = fl32(fl32(x*s) * fl32(1 / fl32(a*s))) with s = 2^64 if a < 2^-64,
 *      s = 2^-64 if a > 2^64, else s = 1.
 *  R4  a non-finite element takes code z = the nearest code to 0.0.
 *  R5  a block with absmax 0 takes code z everywhere.
 *  R6  nearest = exact real distance, ties to the lower index.
 *  R8  4-bit packing: first element of a pair in the high nibble; R9 odd n: pad nibble 0.
 *  R10 fp32 -> fp16/bf16 is round-to-nearest-even, overflow to infinity, signed zeros and
 *      subnormals kept; R15 NaN -> quiet NaN with its sign.
 *  R11 nested mean = RN32(fl64(S / nb)), S the binary64 pairwise sum of the absmax array
 *      zero-padded to a power of two.
 *  R12 statistics: d_b = fl32(a_b - mean), quantized in groups with the 256-entry table;
 *      rebuilt absmax a'_b = fl32(fl32(c2[q2_b] * a2_g) + mean).
 *  R13 GGUF 4-bit block: element j < 16 is the low nibble of byte j, element 16+j its high
 *      nibble; R14 values are (q-8)*d or q*d in binary32 (exact), rounded once.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { BQO_F32 = 0, BQO_F16 = 1, BQO_BF16 = 2 };
enum { BQO_Q4 = 0, BQO_Q8 = 1 };

/* ------------------------------------------------------------------------------------ */
/* IEEE binary16 / bfloat16 <-> binary32, written from the field definitions.            */
/* ------------------------------------------------------------------------------------ */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float bqo_f16_to_f32(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  float mag;
  if (e == 0)
    mag = ldexpf((float)m, -24); /* zero or subnormal: m * 2^-24 */
  else if (e == 31)
    mag = m ? NAN : INFINITY;
  else
    mag = ldexpf((float)(1024 + m), e - 25); /* (1 + m/2^10) * 2^(e-15) */
  return sign ? -mag : mag;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
float bqo_bf16_to_f32(uint16_t b) {
  int sign = b >> 15, e = (b >> 7) & 0xff, m = b & 0x7f;
  float mag;
  if (e == 0)
    mag = ldexpf((float)m, -133); /* zero or subnormal: m * 2^-133 */
  else if (e == 255)
    mag = m ? NAN : INFINITY;
  else
    mag = ldexpf((float)(128 + m), e - 134); /* (1 + m/2^7) * 2^(e-127) */
  return sign ? -mag : mag;
}

/* Round |f| to a floating-point grid with `frac_bits` fraction bits whose smallest normal
 * binade starts at 2^emin; round-to-nearest-even; returns the exact rounded magnitude as a
 * double (which may equal 2^(emax+1), i.e. overflow). */
static double round_to_format(double a, int frac_bits, int emin) {
  int e;
  frexp(a, &e);          /* a in [2^(e-1), 2^e) */
  int E = e - 1;         /* unbiased exponent of a */
  if (E < emin) E = emin; /* subnormals share the quantum of the lowest normal binade */
  double quantum = ldexp(1.0, E - frac_bits);
  return rint(a / quantum) * quantum; /* exact in binary64; rint rounds ties to even */
}

uint16_t bqo_f32_to_bf16(float f) {
  uint16_t sign = signbit(f) ? 0x8000 : 0;
  if (isnan(f)) return sign | 0x7FC0;
  if (isinf(f)) return sign | 0x7F80;
  double a = fabs((double)f);
  if (a == 0.0) return sign;
  double r = round_to_format(a, 7, -126);
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80; /* overflow */
  if (r < ldexp(1.0, -126)) return sign | (uint16_t)(r / ldexp(1.0, -133));
  int e;
  frexp(r, &e);
  int E = e - 1;
  uint16_t m = (uint16_t)(r / ldexp(1.0, E - 7) - 128.0);
  return sign | (uint16_t)((E + 127) << 7) | m;
}

uint16_t bqo_f32_to_f16(float f) {
  uint16_t sign = signbit(f) ? 0x8000 : 0;
  if (isnan(f)) return sign | 0x7E00;
  if (isinf(f)) return sign | 0x7C00;
  double a = fabs((double)f);
  if (a == 0.0) return sign;
  double r = round_to_format(a, 10, -14);
  if (r >= 65536.0) return sign | 0x7C00; /* overflow */
  if (r < ldexp(1.0, -14)) return sign | (uint16_t)(r / ldexp(1.0, -24));
  int e;
  frexp(r, &e);
  int E = e - 1;
  uint16_t m = (uint16_t)(r / ldexp(1.0, E - 10) - 1024.0);
  return sign | (uint16_t)((E + 15) << 10) | m;
}

static float load_elem(const void* in, int dtype, int64_t i) {
  if (dtype == BQO_F32) return ((const float*)in)[i];
  uint16_t h = ((const uint16_t*)in)[i];
  return dtype == BQO_F16 ? bqo_f16_to_f32(h) : bqo_bf16_to_f32(h);
}

static void store_elem(void* out, int dtype, int64_t i, float v) {
  if (dtype == BQO_F32)
    ((float*)out)[i] = v;
  else if (dtype == BQO_F16)
    ((uint16_t*)out)[i] = bqo_f32_to_f16(v);
  else
    ((uint16_t*)out)[i] = bqo_f32_to_bf16(v);
}

/* ------------------------------------------------------------------------------------ */
/* Nearest code (R6).                                                                    */
/* ------------------------------------------------------------------------------------ */

/* Smallest index k minimizing the exact distance |y - c[k]| over an ascending table.
 * For c[j] < c[k], c[k] is strictly closer to y than c[j] exactly when y exceeds their
 * midpoint, i.e. 2y > c[j] + c[k]; equality is a tie, which keeps the lower index
 * (Model-Optimizer IQ packing review, "Search equivalence": lowest index on equal error).
 * Both sides are exact in binary64: 2y only moves the exponent of a binary32 value, and
 * every valid entry is a multiple of 2^-43 of magnitude <= 1, so a sum of two is exact. */
int bqo_nearest(float y, const float* c, int K) {
  int best = 0;
  for (int k = 1; k < K; ++k)
    if (2.0 * (double)y > (double)c[best] + (double)c[k]) best = k;
  return best;
}

/* Code of a non-finite element and of a zero block (R4, R5): the nearest code to 0.0. */
int bqo_zero_code(const float* c, int K) { return bqo_nearest(0.0f, c, K); }

/* Step 1, the code table (R7).  K is 16 or 256; every entry is finite, within [-1, 1], and
 * larger than the one before it; a nonzero entry has magnitude at least 2^-20.  Under these
 * conditions every entry is a multiple of 2^-43 of magnitude at most 1, which is what makes
 * the binary64 midpoint test of bqo_nearest exact.  A -0.0 entry is read as +0.0, the way
 * the IQ packing review treats a negative-zero scale as zero ("[OMNIML-5899] Add CUDA
 * kernels for IQ packing", the later review's negative-zero finding): its code then
 * dequantizes to +0.0.  Writes the table as used into c_out; returns 0, or -1 when the
 * table breaks a condition. */
int bqo_prepare_table(const float* c_in, int K, float* c_out) {
  if (c_in == NULL || (K != 16 && K != 256)) return -1;
  for (int k = 0; k < K; ++k) {
    float v = c_in[k];
    if (!isfinite(v) || v < -1.0f || v > 1.0f) return -1;
    if (v == 0.0f) v = 0.0f; /* -0.0 -> +0.0 */
    if (v != 0.0f && fabsf(v) < 0x1p-20f) return -1;
    if (k > 0 && !(v > c_out[k - 1])) return -1;
    c_out[k] = v;
  }
  return 0;
}

/* Power-of-two guard of R3: keeps fl32(1/(a*s)) a normal, finite binary32 number. */
float bqo_guard_scale(float a) {
  if (a < 0x1p-64f) return 0x1p64f;
  if (a > 0x1p64f) return 0x1p-64f;
  return 1.0f;
}

/* Normalized value of finite x in a block with absmax a > 0 (R3).  Each line is one
 * binary32 operation with its own rounding. */
float bqo_normalize(float x, float a) {
  float s = bqo_guard_scale(a);
  float as = a * s;
  float r = 1.0f / as;
  float xs = x * s;
  float y = xs * r;
  return y;
}

/* ------------------------------------------------------------------------------------ */
/* Blockwise quantize / dequantize (General8 / FP4 / NF4 family; block sizes 32..4096).  */
/* ------------------------------------------------------------------------------------ */

/* Quantizes one block [lo, hi) of `in`; writes its absmax and one code per element. */
static void quantize_block(const void* in, int dtype, int64_t lo, int64_t hi, const float* c,
                           int K, float* absmax_out, uint8_t* codes /* indexed from lo */) {
  int z = bqo_zero_code(c, K);
  float a = 0.0f; /* R2: +0 when the block holds no finite element */
  for (int64_t i = lo; i < hi; ++i) {
    float v = load_elem(in, dtype, i);
    if (isfinite(v) && fabsf(v) > a) a = fabsf(v);
  }
  *absmax_out = a;
  for (int64_t i = lo; i < hi; ++i) {
    float v = load_elem(in, dtype, i);
    if (a == 0.0f || !isfinite(v))
      codes[i - lo] = (uint8_t)z; /* R4, R5 */
    else
      codes[i - lo] = (uint8_t)bqo_nearest(bqo_normalize(v, a), c, K);
  }
}

/* Packs codes[0..n) into `packed`: one byte per code for a 256-entry table, two codes per
 * byte for a 16-entry table with the first of each pair in the high nibble (R8) and a zero
 * pad nibble when n is odd (R9; 33 values -> 17 bytes, as in mobius finding F3). */
static void pack_codes(const uint8_t* codes, int64_t n, int K, uint8_t* packed) {
  if (K == 256) {
    memcpy(packed, codes, (size_t)n);
    return;
  }
  for (int64_t j = 0; j < (n + 1) / 2; ++j) {
    uint8_t hi = codes[2 * j];
    uint8_t lo = (2 * j + 1 < n) ? codes[2 * j + 1] : 0;
    packed[j] = (uint8_t)((hi << 4) | lo);
  }
}

static int unpack_code(const uint8_t* packed, int64_t i, int K) {
  if (K == 256) return packed[i];
  uint8_t byte = packed[i / 2];
  return (i % 2 == 0) ? (byte >> 4) : (byte & 0x0f);
}

static int valid_args(int dtype, int64_t n, int32_t B, int K) {
  if (dtype != BQO_F32 && dtype != BQO_F16 && dtype != BQO_BF16) return 0;
  if (n < 0 || (K != 16 && K != 256)) return 0;
  for (int b = 32; b <= 4096; b *= 2)
    if (B == b) return 1;
  return 0;
}

/* absmax[ceil(n/B)], packed[ceil(n/2) or n]. Returns 0, or -1 on invalid arguments. */
int bqo_quantize_blockwise(const void* in, int dtype, int64_t n, int32_t B, const float* c_in,
                           int K, float* absmax, uint8_t* packed) {
  float c[256];
  if (!valid_args(dtype, n, B, K) || bqo_prepare_table(c_in, K, c) != 0) return -1;
  if (n == 0) return 0;
  uint8_t* codes = (uint8_t*)malloc((size_t)n);
  if (!codes) return -2;
  int64_t nb = (n + B - 1) / B;
  for (int64_t b = 0; b < nb; ++b) {
    int64_t lo = b * B, hi = lo + B < n ? lo + B : n;
    quantize_block(in, dtype, lo, hi, c, K, &absmax[b], codes + lo);
  }
  pack_codes(codes, n, K, packed);
  free(codes);
  return 0;
}

/* out_i = RN_dtype(fl32(c[q_i] * a_b)): one binary32 multiply by the block absmax, one
 * rounding to the output type. */
int bqo_dequantize_blockwise(void* out, int dtype, int64_t n, int32_t B, const float* c_in, int K,
                             const float* absmax, const uint8_t* packed) {
  float c[256];
  if (!valid_args(dtype, n, B, K) || bqo_prepare_table(c_in, K, c) != 0) return -1;
  for (int64_t i = 0; i < n; ++i) {
    float v = c[unpack_code(packed, i, K)] * absmax[i / B];
    store_elem(out, dtype, i, v);
  }
  return 0;
}

/* Fused dequantize + linear, the consumer of A6 (y = x . deq(W)^T): W is the N x K row-major
 * weight tensor quantized blockwise over its flat index (element (n, k) is flat element
 * n*K + k), w = fl32(c[q] * a_b) its binary32 dequantized value (A6 with a binary32 output),
 * and y[m][n] = sum over k of x[m][k] * w[n][k], accumulated in binary64 in ascending k.
 * x is M x K row-major in `dtype`; y is M x N row-major binary64. */
int bqo_linear_blockwise(const void* x, int dtype, int64_t M, int64_t K, int64_t N, int32_t B,
                         const float* c_in, int Kc, const float* absmax, const uint8_t* packed,
                         double* y) {
  float c[256];
  if (M < 0 || K < 0 || N < 0 || !valid_args(dtype, M * K, B, Kc)) return -1;
  if (bqo_prepare_table(c_in, Kc, c) != 0) return -1;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double s = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t flat = n * K + k;
        const float scale = absmax[flat / B];
        const float w = c[unpack_code(packed, flat, Kc)] * scale;
        s += (double)load_elem(x, dtype, m * K + k) * (double)w;
      }
      y[m * N + n] = s;
    }
  return 0;
}

/* Fused dequantize + GEMM with 16-bit weights (the 16-bit-activation, 4-bit-weight GEMM
 * named in stable-diffusion.cpp PR 2278, Summary): each weight is the 16-bit value the
 * dequantize of A6 stores for `dtype` (fp16 or bf16), w16 = RN16(fl32(c[q] * a_b)), and
 * y[m][n] = sum over k of x[m][k] * w16[n][k], accumulated in binary64 in ascending k.  W is
 * the N x K row-major tensor quantized over its flat index; x is M x K row-major in `dtype`;
 * y is M x N row-major binary64. */
int bqo_gemm_blockwise(const void* x, int dtype, int64_t M, int64_t K, int64_t N, int32_t B,
                       const float* c_in, int Kc, const float* absmax, const uint8_t* packed, double* y) {
  float c[256];
  if (dtype == BQO_F32 || M < 0 || K < 0 || N < 0 || !valid_args(dtype, M * K, B, Kc)) return -1;
  if (bqo_prepare_table(c_in, Kc, c) != 0) return -1;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t f = n * K + k;
        const float w32 = c[unpack_code(packed, f, Kc)] * absmax[f / B];
        const float w16 = dtype == BQO_F16 ? bqo_f16_to_f32(bqo_f32_to_f16(w32))
                                           : bqo_bf16_to_f32(bqo_f32_to_bf16(w32));
        acc += (double)load_elem(x, dtype, m * K + k) * (double)w16;
      }
      y[m * N + n] = acc;
    }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Nested statistics (nested General8 / compressed-statistics NF4).                     */
/* ------------------------------------------------------------------------------------ */

/* Binary64 pairwise sum of a[lo .. lo+len) where len is a power of two and entries at or
 * beyond n count as zero (R11): sum(range) = sum(left half) + sum(right half). */
static double pairwise_sum(const float* a, int64_t n, int64_t lo, int64_t len) {
  if (len == 1) return lo < n ? (double)a[lo] : 0.0;
  return pairwise_sum(a, n, lo, len / 2) + pairwise_sum(a, n, lo + len / 2, len / 2);
}

/* S of R11: the binary64 pairwise sum of a[0..n) zero-padded to a power-of-two length. */
double bqo_pairwise_sum(const float* a, int64_t n) {
  int64_t len = 1;
  while (len < n) len *= 2;
  return pairwise_sum(a, n, 0, len);
}

/* Nested mean of R11: RN32(fl64(S / nb)). */
float bqo_nested_mean(const float* absmax, int64_t nb) {
  double S = bqo_pairwise_sum(absmax, nb);
  return (float)(S / (double)nb);
}

/* Statistics of the groups g_lo <= g < g_hi, given the mean (R12): d_b = fl32(a_b - mean) for
 * the blocks of each group of B2 blocks, then the group's maximum |d_b| and the code of each
 * d_b by the same absmax / normalize / nearest rules as the data (R2..R6), with the 256-entry
 * table c2.  Writes q2[b] for the group's blocks and absmax2[g].  Groups are independent, so
 * any split of [0, ceil(nb / B2)) into ranges gives the same outputs. */
int bqo_nested_groups(const float* absmax, int64_t nb, float mean, const float* c2, int K2,
                      int32_t B2, int64_t g_lo, int64_t g_hi, uint8_t* q2, float* absmax2) {
  if (K2 != 256 || !valid_args(BQO_F32, 1, B2, K2) || nb < 0) return -1;
  const int64_t ng = (nb + B2 - 1) / B2;
  if (g_lo < 0 || g_hi > ng || g_lo > g_hi) return -1;
  if (g_lo == g_hi) return 0;
  const int64_t b_lo = g_lo * B2, b_hi = g_hi * B2 < nb ? g_hi * B2 : nb;
  float* d = (float*)malloc((size_t)(b_hi - b_lo) * sizeof(float));
  if (!d) return -2;
  for (int64_t b = b_lo; b < b_hi; ++b) d[b - b_lo] = absmax[b] - mean;
  int rc = bqo_quantize_blockwise(d, BQO_F32, b_hi - b_lo, B2, c2, K2, absmax2 + g_lo, q2 + b_lo);
  free(d);
  return rc;
}

/* The whole second level of the nested statistics: mean = RN32(S / nb) (R11), then every
 * group's q2 and absmax2 (bqo_nested_groups). */
int bqo_nested_stats(const float* absmax, int64_t nb, const float* c2, int K2, int32_t B2,
                     uint8_t* q2, float* absmax2, float* mean) {
  if (nb <= 0) return nb == 0 ? 0 : -1;
  const float m = bqo_nested_mean(absmax, nb);
  *mean = m;
  return bqo_nested_groups(absmax, nb, m, c2, K2, B2, 0, (nb + B2 - 1) / B2, q2, absmax2);
}

/* Quantizes `in` with table c (K entries) and block size B, then quantizes the statistics:
 * d_b = fl32(a_b - mean) in groups of B2 blocks with the 256-entry table c2 (R12), using
 * the same absmax / normalize / nearest rules as the data (R2..R6).
 * Outputs: packed data codes, absmax[nb] (the exact fp32 a_b, an intermediate), q2[nb],
 * absmax2[ceil(nb/B2)], *mean. */
int bqo_quantize_nested(const void* in, int dtype, int64_t n, int32_t B, const float* c, int K,
                        const float* c2, int K2, int32_t B2, float* absmax, uint8_t* q2,
                        float* absmax2, float* mean, uint8_t* packed) {
  float c2p[256];
  if (K2 != 256 || !valid_args(BQO_F32, 1, B2, K2) || bqo_prepare_table(c2, K2, c2p) != 0) return -1;
  int rc = bqo_quantize_blockwise(in, dtype, n, B, c, K, absmax, packed);
  if (rc != 0 || n == 0) return rc;
  return bqo_nested_stats(absmax, (n + B - 1) / B, c2, K2, B2, q2, absmax2, mean);
}

/* Rebuilt absmax a'_b = fl32(fl32(c2[q2_b] * a2_g) + mean), then the blockwise dequantize
 * with a'_b. */
int bqo_dequantize_nested(void* out, int dtype, int64_t n, int32_t B, const float* c, int K,
                          const float* c2_in, int K2, int32_t B2, const uint8_t* q2,
                          const float* absmax2, float mean, const uint8_t* packed) {
  float c2[256];
  if (K2 != 256 || !valid_args(BQO_F32, 1, B2, K2) || bqo_prepare_table(c2_in, K2, c2) != 0) return -1;
  if (!valid_args(dtype, n, B, K)) return -1;
  int64_t nb = (n + B - 1) / B;
  float* a = (float*)malloc((size_t)(nb ? nb : 1) * sizeof(float));
  if (!a) return -2;
  for (int64_t b = 0; b < nb; ++b) {
    float scaled = c2[q2[b]] * absmax2[b / B2];
    a[b] = scaled + mean;
  }
  int rc = bqo_dequantize_blockwise(out, dtype, n, B, c, K, a, packed);
  free(a);
  return rc;
}

/* ------------------------------------------------------------------------------------ */
/* GGUF-style 32-element blocks (Q4_0 / Q8_0 shapes of "Cache device-side constants in    */
/* dequant kernels").                                                                    */
/* ------------------------------------------------------------------------------------ */

/* blocks: n/32 consecutive blocks of 18 bytes (Q4: fp16 d little-endian, 16 bytes of
 * nibbles) or 34 bytes (Q8: fp16 d, 32 int8).  Q4 element j < 16 is the low nibble of byte
 * j and element 16+j the high nibble (R13), value (q-8)*d; Q8 value q*d.  The binary32
 * product is exact (at most 5 x 11 or 8 x 11 significant bits), then rounded once (R14).
 * row_len must be a multiple of 32 dividing n (rows never split a block). */
int bqo_dequant_q32(const uint8_t* blocks, int dtype, int64_t n, int32_t row_len, int fmt,
                    void* out) {
  if (dtype != BQO_F32 && dtype != BQO_F16 && dtype != BQO_BF16) return -1;
  if (fmt != BQO_Q4 && fmt != BQO_Q8) return -1;
  if (row_len <= 0 || row_len % 32 != 0 || n < 0 || n % row_len != 0) return -1;
  int64_t nblk = n / 32;
  int bsize = fmt == BQO_Q4 ? 18 : 34;
  for (int64_t b = 0; b < nblk; ++b) {
    const uint8_t* blk = blocks + b * bsize;
    float d = bqo_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
    if (fmt == BQO_Q4) {
      for (int j = 0; j < 16; ++j) {
        int lo = blk[2 + j] & 0x0f, hi = blk[2 + j] >> 4;
        store_elem(out, dtype, b * 32 + j, (float)(lo - 8) * d);
        store_elem(out, dtype, b * 32 + 16 + j, (float)(hi - 8) * d);
      }
    } else {
      for (int j = 0; j < 32; ++j) {
        int q = (int8_t)blk[2 + j];
        store_elem(out, dtype, b * 32 + j, (float)q * d);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* IQ2_XS-style search encoding and its decoding ("[OMNIML-5899] Add CUDA kernels for IQ  */
/* packing", Model-Optimizer PR 2448: the Summary, "Dependency behavior", and the review   */
/* items "Wire format", "Scale anchors", "Even-parity sign field", "Search equivalence";   */
/* the later review's "IQ2_XS grouping" and "Negative scales" replies).                    */
/*                                                                                        */
/* Superblock: 256 consecutive elements, 74 bytes:                                        */
/*   bytes 0-1   the caller's binary16 scale d (little-endian);                           */
/*   bytes 2-65  32 little-endian 16-bit words, one per 8-element vector v (elements        */
/*               8v .. 8v+7): bits 0-8 the grid entry e, bits 9-15 the signs of elements    */
/*               0-6 (bit set = negative); element 7's sign makes the count even;          */
/*   bytes 66-73 byte i = ls[2i] | ls[2i+1] << 4, ls[g] the 4-bit local scale of group g    */
/*               (elements 16g .. 16g+15, vectors 2g and 2g+1).                             */
/* Decoded element j of vector v: d * (2*ls + 1) / 8 * grid[e][j] * (-1 if its sign bit).   */
/* The grid (512 entries of 8 magnitude bytes) is the caller's: the pages do not hold it.   */
/*                                                                                        */
/* Readings (restated where used):                                                        */
/*  I1 a non-finite element is read as +0.0 (the Summary normalizes non-finite inputs);    */
/*     -0.0 counts as non-negative.                                                        */
/*  I2 d with no magnitude bits (+0.0 or -0.0) gives the all-zero payload; a NaN, infinite  */
/*     or negative d is rejected (counted) and also gets the all-zero payload.             */
/*  I3 a vector's error for entry e at scale s is the pages' clamped form                   */
/*     max(fma(s*s, qn, fma(-2s, dot, xn)), 0) in binary32: xn = fma-chain sum of a_j^2,     */
/*     dot = fma-chain sum of a_j*q_j (j ascending, from +0), qn = sum of q_j^2 (exact),    */
/*     a_j = |x_j|; with an odd count of negative elements, dot becomes fma(-2, w, dot),    */
/*     w = min_j fl(a_j*q_j), and the sign of the first element reaching w is flipped.     */
/*  I4 s = d*(2*ls+1)/8 (exact in binary32).  Each group takes the local scale whose       */
/*     summed error fl(E(v0) + E(v1)) is least, E(v) = min over entries of the error;       */
/*     equal sums go to the lower ls.  Each vector then takes the entry of least error at   */
/*     that scale, equal errors to the lower entry index.                                   */
/* ------------------------------------------------------------------------------------ */

enum { IQ_BLOCK = 256, IQ_VEC = 8, IQ_ENTRIES = 512, IQ_BYTES = 74 };

typedef struct {
  float a[IQ_VEC]; /* |x_j| (I1) */
  int neg;         /* bit j set: x_j < 0 */
  int odd;         /* odd count of negative elements */
  float xn;        /* fma-chain sum of a_j^2 */
} iq_vector;

static void iq_load_vector(const float* x, iq_vector* v) {
  v->neg = 0;
  v->xn = 0.0f;
  int count = 0;
  for (int j = 0; j < IQ_VEC; ++j) {
    float t = isfinite(x[j]) ? x[j] : 0.0f; /* I1 */
    if (t < 0.0f) {
      v->neg |= 1 << j;
      ++count;
    }
    v->a[j] = fabsf(t);
  }
  v->odd = count & 1;
  for (int j = 0; j < IQ_VEC; ++j) v->xn = fmaf(v->a[j], v->a[j], v->xn);
}

/* dot of |x| with the entry's magnitudes, after the even-parity correction (I3); *flip is
 * the element whose sign the correction flips, or -1. */
static float iq_entry_dot(const iq_vector* v, const uint8_t* q, int* flip) {
  float dot = 0.0f;
  for (int j = 0; j < IQ_VEC; ++j) dot = fmaf(v->a[j], (float)q[j], dot);
  *flip = -1;
  if (v->odd) {
    int k = 0;
    float w = v->a[0] * (float)q[0];
    for (int j = 1; j < IQ_VEC; ++j) {
      float p = v->a[j] * (float)q[j];
      if (p < w) {
        w = p;
        k = j;
      }
    }
    dot = fmaf(-2.0f, w, dot);
    *flip = k;
  }
  return dot;
}

static float iq_entry_qnorm(const uint8_t* q) {
  float s = 0.0f;
  for (int j = 0; j < IQ_VEC; ++j) s += (float)q[j] * (float)q[j]; /* integers, exact */
  return s;
}

/* The clamped error of I3 at scale s. */
float iqo_vector_error(float xn, float dot, float qn, float s) {
  return fmaxf(fmaf(s * s, qn, fmaf(-2.0f * s, dot, xn)), 0.0f);
}

/* Least error over the grid at scale s (I4); *entry gets the lowest index reaching it. */
static float iq_best_entry(const iq_vector* v, const uint8_t* grid, float s, int* entry) {
  float best = 0.0f;
  for (int e = 0; e < IQ_ENTRIES; ++e) {
    int flip;
    const uint8_t* q = grid + IQ_VEC * e;
    float err = iqo_vector_error(v->xn, iq_entry_dot(v, q, &flip), iq_entry_qnorm(q), s);
    if (e == 0 || err < best) {
      best = err;
      *entry = e;
    }
  }
  return best;
}

/* Encodes one superblock of 256 binary32 values; returns 1 when d is rejected (I2). */
int iqo_iq2xs_encode_block(const float* x, uint16_t d_bits, const uint8_t* grid, uint8_t* out) {
  memset(out, 0, IQ_BYTES);
  if ((d_bits & 0x7fff) == 0) return 0;                             /* I2: zero scale */
  if ((d_bits & 0x7c00) == 0x7c00 || (d_bits & 0x8000)) return 1;   /* I2: NaN, inf, negative */
  float d = bqo_f16_to_f32(d_bits);
  out[0] = (uint8_t)(d_bits & 0xff);
  out[1] = (uint8_t)(d_bits >> 8);
  iq_vector vec[IQ_BLOCK / IQ_VEC];
  for (int v = 0; v < IQ_BLOCK / IQ_VEC; ++v) iq_load_vector(x + IQ_VEC * v, &vec[v]);
  int ls[16];
  for (int g = 0; g < 16; ++g) {
    int best_l = 0;
    float best_sum = 0.0f;
    for (int l = 0; l < 16; ++l) {
      float s = d * (float)(2 * l + 1) * 0.125f; /* I4 */
      int e0, e1;
      float sum = iq_best_entry(&vec[2 * g], grid, s, &e0) + iq_best_entry(&vec[2 * g + 1], grid, s, &e1);
      if (l == 0 || sum < best_sum) {
        best_sum = sum;
        best_l = l;
      }
    }
    ls[g] = best_l;
    float s = d * (float)(2 * best_l + 1) * 0.125f;
    for (int v = 2 * g; v < 2 * g + 2; ++v) {
      int e = 0, flip;
      iq_best_entry(&vec[v], grid, s, &e);
      iq_entry_dot(&vec[v], grid + IQ_VEC * e, &flip);
      int signs = vec[v].neg ^ (flip >= 0 ? 1 << flip : 0); /* even count of set bits */
      uint16_t word = (uint16_t)(e | ((signs & 0x7f) << 9));
      out[2 + 2 * v] = (uint8_t)(word & 0xff);
      out[3 + 2 * v] = (uint8_t)(word >> 8);
    }
  }
  for (int i = 0; i < 8; ++i) out[66 + i] = (uint8_t)(ls[2 * i] | (ls[2 * i + 1] << 4));
  return 0;
}

/* Superblocks [b_lo, b_hi) of an n-element input of `dtype` (n a multiple of 256); returns
 * the number of rejected scales, or -1 for invalid arguments. */
int64_t iqo_iq2xs_quantize(const void* in, int dtype, int64_t n, const uint8_t* grid,
                           const uint16_t* scales, uint8_t* out, int64_t b_lo, int64_t b_hi) {
  if (dtype != BQO_F32 && dtype != BQO_F16 && dtype != BQO_BF16) return -1;
  if (n < 0 || n % IQ_BLOCK != 0 || b_lo < 0 || b_hi > n / IQ_BLOCK) return -1;
  int64_t rejected = 0;
  float x[IQ_BLOCK];
  for (int64_t b = b_lo; b < b_hi; ++b) {
    for (int i = 0; i < IQ_BLOCK; ++i) x[i] = load_elem(in, dtype, b * IQ_BLOCK + i);
    rejected += iqo_iq2xs_encode_block(x, scales[b], grid, out + b * IQ_BYTES);
  }
  return rejected;
}

/* Decodes n/256 superblocks to `dtype`: the binary32 value d*(2*ls+1)/8*q is exact (11, 5
 * and 8 significant bits), then rounded once (R10); the sign is a negation. */
int iqo_iq2xs_dequantize(const uint8_t* blocks, const uint8_t* grid, int64_t n, int dtype, void* out) {
  if (dtype != BQO_F32 && dtype != BQO_F16 && dtype != BQO_BF16) return -1;
  if (n < 0 || n % IQ_BLOCK != 0) return -1;
  for (int64_t b = 0; b < n / IQ_BLOCK; ++b) {
    const uint8_t* blk = blocks + b * IQ_BYTES;
    float d = bqo_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
    for (int v = 0; v < IQ_BLOCK / IQ_VEC; ++v) {
      int g = v / 2;
      int ls = (blk[66 + g / 2] >> (4 * (g % 2))) & 0xf;
      float dl = d * (float)(2 * ls + 1) * 0.125f;
      int word = blk[2 + 2 * v] | (blk[3 + 2 * v] << 8);
      int e = word & 0x1ff, signs = word >> 9, parity = 0;
      for (int j = 0; j < 7; ++j) parity ^= (signs >> j) & 1;
      signs |= parity << 7;
      for (int j = 0; j < IQ_VEC; ++j) {
        float val = dl * (float)grid[IQ_VEC * e + j];
        store_elem(out, dtype, b * IQ_BLOCK + IQ_VEC * v + j, ((signs >> j) & 1) ? -val : val);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* IQ1_S-style encoding and its decoding ("[OMNIML-5899] Add CUDA kernels for IQ packing", */
/* Model-Optimizer PR 2448: the Summary, "Provenance" (16.875 = 15 x (1 + 1/8), 0.61, the   */
/* 0.125 delta), the review items "Wire format", "Scale anchors", "Search equivalence", the */
/* round-3 "IQ1_S shifted objective" item and the reply on the shared helpers (qsum, the   */
/* 8*delta^2 term)).                                                                        */
/*                                                                                        */
/* Superblock: 256 consecutive elements, 50 bytes:                                        */
/*   bytes 0-1   binary16 scale d (little-endian);                                        */
/*   bytes 2-33  qs[v] = the low 8 bits of vector v's 11-bit grid entry;                   */
/*   bytes 34-49 8 little-endian 16-bit words qh[b], one per 32-element sub-block b (vectors */
/*               4b .. 4b+3): bits 3l..3l+2 the high 3 bits of vector 4b+l's entry, bits    */
/*               12-14 the local scale ls, bit 15 the delta sign (set: delta = -1/8).       */
/* Decoded element j of vector v: fl32(d * (2 ls + 1) * fl32(g_j + delta)), g = the grid's  */
/* signed byte (the IQ1_S grid is ternary: -1, 0, +1, where the product is exact).          */
/* The grid (2048 entries of 8 signed bytes) is the caller's: the pages do not hold it.    */
/*                                                                                        */
/* Readings (restated where used):                                                        */
/*  J1 non-finite elements read as +0.0 (as I1).                                           */
/*  J2 the scale: amax = the largest |x| over the superblock (from +0), then              */
/*     d = RN16(fl32(fl32(amax / 16.875) * 0.61)), saturated to the largest finite binary16;  */
/*     a d with no magnitude bits gives the all-zero superblock.                            */
/*  J3 a vector's error for entry e and choice (ls, sign), dl = d * (2 ls + 1) (exact),     */
/*     delta = +-1/8: xn = fma-chain sum of x_j^2, dot = fma-chain sum of x_j * g_j, xsum =   */
/*     fma-chain sum of x_j * 1 (all j ascending from +0); sdot = fma(delta, xsum, dot);     */
/*     snorm = qn + 2 delta qs + 8 delta^2 (qn = sum g^2, qs = sum g: exact);              */
/*     error = max(fma(dl * dl, snorm, fma(-2 dl, sdot, xn)), 0).                           */
/*  J4 each sub-block takes the choice c = ls + 8 * sign (0..15) of least summed error over  */
/*     its four vectors (sums in vector order; equal sums: the lower c), then each vector  */
/*     the entry of least error at that choice (equal errors: the lower entry).            */
/* ------------------------------------------------------------------------------------ */

enum { IQ1_ENTRIES = 2048, IQ1_BYTES = 50 };

/* J2: the superblock scale from its largest magnitude. */
uint16_t iqo_iq1s_scale(float amax) {
  float d = (amax / 16.875f) * 0.61f;
  uint16_t h = bqo_f32_to_f16(d);
  if ((h & 0x7c00) == 0x7c00) h = 0x7bff; /* saturate (amax is finite and >= 0) */
  return h;
}

static float iq1_error(float xn, float dot, float xsum, float qn, float qs, float dl, float delta) {
  float sdot = fmaf(delta, xsum, dot);
  float snorm = qn + 2.0f * delta * qs + 8.0f * delta * delta; /* exact */
  return fmaxf(fmaf(dl * dl, snorm, fmaf(-2.0f * dl, sdot, xn)), 0.0f);
}

/* Least error of a vector over the grid at choice (dl, delta); *entry gets the lowest index. */
static float iq1_best_entry(const float* x, float xn, float xsum, const int8_t* grid, float dl, float delta,
                            int* entry) {
  float best = 0.0f;
  for (int e = 0; e < IQ1_ENTRIES; ++e) {
    const int8_t* g = grid + IQ_VEC * e;
    float dot = 0.0f, qn = 0.0f, qs = 0.0f;
    for (int j = 0; j < IQ_VEC; ++j) {
      dot = fmaf(x[j], (float)g[j], dot);
      qn += (float)g[j] * (float)g[j];
      qs += (float)g[j];
    }
    float err = iq1_error(xn, dot, xsum, qn, qs, dl, delta);
    if (e == 0 || err < best) {
      best = err;
      *entry = e;
    }
  }
  return best;
}

/* Encodes one superblock of 256 binary32 values. */
void iqo_iq1s_encode_block(const float* x_in, const int8_t* grid, uint8_t* out) {
  float x[IQ_BLOCK], amax = 0.0f;
  for (int i = 0; i < IQ_BLOCK; ++i) {
    x[i] = isfinite(x_in[i]) ? x_in[i] : 0.0f; /* J1 */
    amax = fmaxf(amax, fabsf(x[i]));
  }
  memset(out, 0, IQ1_BYTES);
  const uint16_t d_bits = iqo_iq1s_scale(amax);
  if ((d_bits & 0x7fff) == 0) return; /* J2: zero superblock */
  const float d = bqo_f16_to_f32(d_bits);
  out[0] = (uint8_t)(d_bits & 0xff);
  out[1] = (uint8_t)(d_bits >> 8);
  for (int b = 0; b < 8; ++b) {
    float xn[4], xsum[4];
    for (int l = 0; l < 4; ++l) {
      const float* v = x + 32 * b + 8 * l;
      xn[l] = 0.0f;
      xsum[l] = 0.0f;
      for (int j = 0; j < IQ_VEC; ++j) {
        xn[l] = fmaf(v[j], v[j], xn[l]);
        xsum[l] = fmaf(v[j], 1.0f, xsum[l]);
      }
    }
    int best_c = 0;
    float best_sum = 0.0f;
    for (int c = 0; c < 16; ++c) { /* J4 */
      const float dl = d * (float)(2 * (c & 7) + 1), delta = (c & 8) ? -0.125f : 0.125f;
      float sum = 0.0f;
      for (int l = 0; l < 4; ++l) {
        int e;
        sum += iq1_best_entry(x + 32 * b + 8 * l, xn[l], xsum[l], grid, dl, delta, &e);
      }
      if (c == 0 || sum < best_sum) {
        best_sum = sum;
        best_c = c;
      }
    }
    const float dl = d * (float)(2 * (best_c & 7) + 1), delta = (best_c & 8) ? -0.125f : 0.125f;
    uint32_t qh = (uint32_t)(best_c & 7) << 12 | (uint32_t)(best_c >> 3) << 15;
    for (int l = 0; l < 4; ++l) {
      int e = 0;
      iq1_best_entry(x + 32 * b + 8 * l, xn[l], xsum[l], grid, dl, delta, &e);
      out[2 + 4 * b + l] = (uint8_t)(e & 0xff);
      qh |= (uint32_t)(e >> 8) << (3 * l);
    }
    out[34 + 2 * b] = (uint8_t)(qh & 0xff);
    out[35 + 2 * b] = (uint8_t)(qh >> 8);
  }
}

/* Superblocks [b_lo, b_hi) of an n-element input of `dtype` (n a multiple of 256). */
int iqo_iq1s_quantize(const void* in, int dtype, int64_t n, const int8_t* grid, uint8_t* out, int64_t b_lo,
                      int64_t b_hi) {
  if (dtype != BQO_F32 && dtype != BQO_F16 && dtype != BQO_BF16) return -1;
  if (n < 0 || n % IQ_BLOCK != 0 || b_lo < 0 || b_hi > n / IQ_BLOCK) return -1;
  float x[IQ_BLOCK];
  for (int64_t b = b_lo; b < b_hi; ++b) {
    for (int i = 0; i < IQ_BLOCK; ++i) x[i] = load_elem(in, dtype, b * IQ_BLOCK + i);
    iqo_iq1s_encode_block(x, grid, out + b * IQ1_BYTES);
  }
  return 0;
}

/* Decodes n/256 superblocks to `dtype`: fl32(fl32(d * (2 ls + 1)) * fl32(g + delta)), both
 * inner values exact, then rounded once (R10). */
int iqo_iq1s_dequantize(const uint8_t* blocks, const int8_t* grid, int64_t n, int dtype, void* out) {
  if (dtype != BQO_F32 && dtype != BQO_F16 && dtype != BQO_BF16) return -1;
  if (n < 0 || n % IQ_BLOCK != 0) return -1;
  for (int64_t b = 0; b < n / IQ_BLOCK; ++b) {
    const uint8_t* blk = blocks + b * IQ1_BYTES;
    const float d = bqo_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
    for (int sb = 0; sb < 8; ++sb) {
      const int qh = blk[34 + 2 * sb] | (blk[35 + 2 * sb] << 8);
      const float dl = d * (float)(2 * ((qh >> 12) & 7) + 1);
      const float delta = (qh & 0x8000) ? -0.125f : 0.125f;
      for (int l = 0; l < 4; ++l) {
        const int e = blk[2 + 4 * sb + l] | (((qh >> (3 * l)) & 7) << 8);
        for (int j = 0; j < IQ_VEC; ++j) {
          const float y = (float)grid[IQ_VEC * e + j] + delta;
          store_elem(out, dtype, b * IQ_BLOCK + 32 * sb + 8 * l + j, dl * y);
        }
      }
    }
  }
  return 0;
}
