/*
 * bq_oracle.c -- CPU oracle for blockwise absmax quantization and dequantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, scalar definition of what the
 * GPU library computes.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the library itself never does.  It shares no code, header,
 * table or constant generator with the GPU path.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (binary32 operations round once each, round-to-nearest-even; no fused multiply-add).
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
int bqo_quantize_blockwise(const void* in, int dtype, int64_t n, int32_t B, const float* c,
                           int K, float* absmax, uint8_t* packed) {
  if (!valid_args(dtype, n, B, K)) return -1;
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
int bqo_dequantize_blockwise(void* out, int dtype, int64_t n, int32_t B, const float* c, int K,
                             const float* absmax, const uint8_t* packed) {
  if (!valid_args(dtype, n, B, K)) return -1;
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
                         const float* c, int Kc, const float* absmax, const uint8_t* packed,
                         double* y) {
  if (M < 0 || K < 0 || N < 0 || !valid_args(dtype, M * K, B, Kc)) return -1;
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
                       const float* c, int Kc, const float* absmax, const uint8_t* packed, double* y) {
  if (dtype == BQO_F32 || M < 0 || K < 0 || N < 0 || !valid_args(dtype, M * K, B, Kc)) return -1;
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

/* Quantizes `in` with table c (K entries) and block size B, then quantizes the statistics:
 * d_b = fl32(a_b - mean) in groups of B2 blocks with the 256-entry table c2 (R12), using
 * the same absmax / normalize / nearest rules as the data (R2..R6).
 * Outputs: packed data codes, absmax[nb] (the exact fp32 a_b, an intermediate), q2[nb],
 * absmax2[ceil(nb/B2)], *mean. */
int bqo_quantize_nested(const void* in, int dtype, int64_t n, int32_t B, const float* c, int K,
                        const float* c2, int K2, int32_t B2, float* absmax, uint8_t* q2,
                        float* absmax2, float* mean, uint8_t* packed) {
  if (K2 != 256 || !valid_args(BQO_F32, 1, B2, K2)) return -1;
  int rc = bqo_quantize_blockwise(in, dtype, n, B, c, K, absmax, packed);
  if (rc != 0 || n == 0) return rc;
  int64_t nb = (n + B - 1) / B;
  float m = bqo_nested_mean(absmax, nb);
  *mean = m;
  float* d = (float*)malloc((size_t)nb * sizeof(float));
  if (!d) return -2;
  for (int64_t b = 0; b < nb; ++b) d[b] = absmax[b] - m;
  rc = bqo_quantize_blockwise(d, BQO_F32, nb, B2, c2, K2, absmax2, q2);
  free(d);
  return rc;
}

/* Rebuilt absmax a'_b = fl32(fl32(c2[q2_b] * a2_g) + mean), then the blockwise dequantize
 * with a'_b. */
int bqo_dequantize_nested(void* out, int dtype, int64_t n, int32_t B, const float* c, int K,
                          const float* c2, int K2, int32_t B2, const uint8_t* q2,
                          const float* absmax2, float mean, const uint8_t* packed) {
  if (K2 != 256 || !valid_args(BQO_F32, 1, B2, K2)) return -1;
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
