// bq_internal.h -- definitions shared by the host layer and the gfx950 kernels of libbq.
//
// Nearest-code search on the GPU.  For an ascending table c_0 < ... < c_{K-1} the host
// builds thresholds T_k = the smallest binary32 value strictly greater than the midpoint
// (c_k + c_{k+1}) / 2 (exact in binary64 for valid tables).  For a binary32 y, y > midpoint
// exactly when y >= T_k, so the nearest index with ties to the lower index is
//     q(y) = #{ k : y >= T_k }.
// A monotone "bucket" function of y selects a small LUT entry holding base = #{k : T_k lies
// in a lower bucket} and the next M thresholds; then q = base + sum_m [y >= t_m].  Values
// whose bucket holds no threshold need no compare at all.  Non-finite y (non-finite input,
// or 0 * inf in a zero block) land in "special" buckets whose entry is (z, NaN, NaN, ...):
// every compare with NaN is false, so they take the zero code z.
#pragma once

#include <stdint.h>

namespace bq {

enum Dtype : int { F32 = 0, F16 = 1, BF16 = 2 };

// Bucket functions (MODE):
//   LIN:    zz = clamp(fma(y, 31/128, 3/4), 0, 1);  idx = bits(zz)[23:SH]
//           Finite y in [-1, 1] gives zz in [0.5078125, 0.9921875], so idx in (0, H) with
//           H = 2^(23-SH); NaN and -inf clamp to 0 (idx 0), +inf to 1.0 (idx H).  Uniform
//           buckets in y: right for tables of roughly even spacing.
//   LOG:    a = bits(y) & 0x7fffffff;  j = (min(max(a, LO), HI) - LO) >> SH;
//           idx = j + (sign(y) ? NJ : 0).  2^(23-SH) buckets per octave of |y| between
//           2^-E and 1; j = NJ-1 (a >= HI) only for non-finite y.  Right for tables that
//           are dense near 0.
//   SEARCH: no buckets; branchless binary search over T (any valid table).
enum Mode : int { LIN = 0, LOG = 1, SEARCH = 2 };

constexpr float kLinAlpha = 0.2421875f;  // 31/128
constexpr float kLinBeta = 0.75f;
constexpr int kLutMax = 2100;            // LUT entries carried in the kernel arguments
constexpr int kLinLutMax = 513;          // uniform buckets: H <= 512, plus the +inf bucket

struct QuantArgs {
  // Table-derived data (built on the host per call, passed by value).
  float thr[260];           // T_0..T_{K-2}, then NaN padding
  uint8_t base[kLutMax];    // per bucket: number of thresholds in lower buckets
  int32_t nbuckets;
  int32_t special0, special1;  // the two special bucket indices (non-finite y)
  int32_t z;                // code of 0.0
  int32_t K;
  // Bucket parameters.
  int32_t sh;               // LIN and LOG shift
  uint32_t lo, hi;          // LOG clamp bounds (bit patterns of |y|)
  int32_t nj;               // LOG buckets per sign
  // LOG, as the kernels evaluate it: LUT byte offset = (clamp(|y| bits >> SH, jlo, jhi) << log2
  // of the entry size) + (y negative ? log_nbias : log_bias), in modulo-2^32 arithmetic.
  uint32_t jlo, jhi;        // LO >> SH, HI >> SH
  uint32_t log_bias;        // -(jlo * entry size)
  uint32_t log_nbias;       // log_bias + NJ * entry size
};

struct DequantArgs {
  float c[256];
  int32_t K;
};

struct NestedDequantArgs {
  float c[256];   // data table
  float c2[256];  // statistics table
  int32_t K;
};

// Host-side table preparation (bq_table.cpp).
struct PreparedTable {
  QuantArgs qa;
  int mode;   // Mode
  int M;      // compares per element (LIN / LOG)
  float c[256];
  int K;
};

// Returns false when the table violates the documented preconditions.
bool prepare_table(const float* entries, int size, PreparedTable* out);

// The bucket function, evaluated identically on host and device (integer ops on bit
// patterns and one correctly rounded fma).
#if defined(__HIPCC__)
#define BQ_HD __host__ __device__ __forceinline__
#else
#define BQ_HD inline
#endif

BQ_HD uint32_t f32_bits(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  return v.u;
}

BQ_HD float bits_f32(uint32_t u) {
  union { float f; uint32_t u; } v;
  v.u = u;
  return v.f;
}

}  // namespace bq

// Launchers (k_*.hip).  Each returns the hipError_t of its launches as an int.
namespace bq {
// Fused dequantize + linear for M <= 4 (k_linear.hip): y (M x N, binary32) = x . deq(W)^T.
int launch_linear(const void* x, int dtype, int64_t M, int64_t K, int64_t N, int blocksize, const DequantArgs& da,
                  const float* absmax, const uint8_t* packed, float* y, void* stream);

// Fused dequantize + GEMM on MFMA (k_gemm.hip): y (M x N, binary32) = x . W16^T, x bf16/fp16.
int launch_gemm(const void* x, int dtype, int64_t M, int64_t K, int64_t N, int blocksize, const DequantArgs& da,
                const float* absmax, const uint8_t* packed, float* y, void* stream);

int launch_quantize(const void* in, int dtype, int64_t n, int blocksize, const PreparedTable& t,
                    float* absmax, uint8_t* packed, double* partials, void* stream);
// Workgroups of a quantize launch over n elements.
int quantize_grid(int64_t n);
// Partial sums a quantize launch writes: one per wave of 2048 elements (one per pair of waves
// for B = 4096, whose blocks span two waves), including waves past n, which write +0.
int64_t quantize_partials(int64_t n, int blocksize);
constexpr int64_t kQuantTileElems = 8192;  // elements per quantize tile
int launch_dequantize(void* out, int dtype, int64_t n, int blocksize, const DequantArgs& a,
                      const float* absmax, const uint8_t* packed, void* stream);
int launch_nested_stats(const float* absmax, int64_t nb, int blocksize2, const PreparedTable& t2,
                        double* partials, int64_t npart, uint8_t* q2, float* absmax2, float* mean,
                        void* stream);
int launch_dequantize_nested(void* out, int dtype, int64_t n, int blocksize, int blocksize2,
                             const NestedDequantArgs& a, const uint8_t* q2, const float* absmax2,
                             const float* mean, const uint8_t* packed, void* stream);
int launch_q32(const void* blocks, int dtype, int64_t n, int fmt, void* out, void* stream);
}  // namespace bq
