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

// Bucket functions (MODE), for y in [-1, 1] (the kernels bring a non-finite element, or the
// elements of a zero block, to y = 0, whose code is z):
//   LIN:    zz = fma(y, H/2, 2^23 + H/2), rounded to nearest, is an integer in [2^23, 2^23 + H]
//           (the binary32 values of [2^23, 2^24) are the integers), so bits(zz) = 0x4B000000 +
//           idx with idx in [0, H]: H + 1 uniform buckets of width 2/H in y, and the entry's
//           byte offset is one shift-and-add of bits(zz).  Right for tables of roughly even
//           spacing.
//   LOG:    a = bits(y) & 0x7fffffff;  j = (min(max(a, LO), HI) - LO) >> SH;
//           idx = j + (sign(y) ? NJ : 0).  2^(23-SH) buckets per octave of |y| between
//           2^-E and 1; j = NJ-1 (a >= HI) only for non-finite y.  Right for tables that
//           are dense near 0.
//   F16B:   h = the binary16 bits of y rounded toward zero (v_cvt_pkrtz_f16_f32, two elements
//           per instruction); for |y| <= 1 bit 14 of h is clear, so moving the sign (bit 15)
//           there, h' = (h & 0x3ff0) | ((h & 0x8000) >> 1), and idx = h' >> 4 give 64 buckets
//           per octave of |y| from 2^-14 to 1, linear ones below, and every |y| < 2^-24 in the
//           bucket of its signed zero.  Positive y give idx 0..960, negative y 1024..1984, so
//           the LUT has 1985 entries with a small hole at 961..1023, and two elements' byte
//           offsets take six operations.  The host keeps the bases of the two halves side by
//           side (base index idx, or idx - 63 for negative y).  Right for tables that are dense
//           near 0, with one compare.
//   SEARCH: no buckets; branchless binary search over T (any valid table).
enum Mode : int { LIN = 0, LOG = 1, SEARCH = 2, F16B = 3 };
constexpr int kF16Pos = 961;       // F16B buckets of positive y: 0 .. 960
constexpr int kF16NegLo = 1024;    // F16B buckets of negative y: 1024 .. 1984
constexpr int kF16Size = 1985;     // F16B LUT entries, the hole 961 .. 1023 included
constexpr int kF16NegBase = kF16NegLo - kF16Pos;  // 63: base index of negative bucket idx is idx - 63

constexpr int kLutMax = 2100;            // LUT entries carried in the kernel arguments
constexpr int kLinLutMax = 513;          // uniform buckets: H <= 512, so at most 513 entries
constexpr uint32_t kLinBits = 0x4B000000u;  // bits of 2^23

struct QuantArgs {
  // Table-derived data (built on the host per call, passed by value).
  float thr[260];           // T_0..T_{K-2}, then NaN padding
  uint8_t base[kLutMax];    // per bucket: number of thresholds in lower buckets
  int32_t nbuckets;
  int32_t special0, special1;  // the two special bucket indices (non-finite y)
  int32_t z;                // code of 0.0
  int32_t K;
  // Bucket parameters.
  float lin_scale, lin_bias;  // LIN: H / 2 and 2^23 + H / 2
  uint32_t lin_off;         // LIN: LUT byte offset = (bits(zz) << log2 of the entry size) + lin_off
  int32_t sh;               // LOG shift
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
// Set when the launcher itself refuses a grid of more than 2^32 - 1 threads (it then returns
// hipErrorInvalidConfiguration without calling HIP); the C ABI layer reads and clears it, so
// that this refusal is told apart from the same error coming from the runtime.
inline thread_local bool g_launch_refused_for_size = false;
// Events (hipEvent_t) that the next kernel launch on this thread stamps with that kernel's own
// start and end time (hipExtLaunchKernel), then forgets.  Set only by the measurement hook of
// bq_debug.h.
inline thread_local void* g_next_launch_start = nullptr;
inline thread_local void* g_next_launch_stop = nullptr;

// Fused dequantize + linear for M <= 4 (k_linear.hip): y (M x N, binary32) = x . deq(W)^T.
int launch_linear(const void* x, int dtype, int64_t M, int64_t K, int64_t N, int blocksize, const DequantArgs& da,
                  const float* absmax, const uint8_t* packed, float* y, void* stream);

// Fused dequantize + GEMM on MFMA (k_gemm.hip): y (M x N, binary32) = x . W16^T, x bf16/fp16.
int launch_gemm(const void* x, int dtype, int64_t M, int64_t K, int64_t N, int blocksize, const DequantArgs& da,
                const float* absmax, const uint8_t* packed, float* y, void* stream);

// Quantize kernel launch.  nested == false: binary32 block maxima into absmax.  nested == true
// (the data pass of a nested quantize): the block maxima in the input's own format (binary32
// for fp32 input, the 16-bit pattern for fp16 / bf16 input).
int launch_quantize(const void* in, int dtype, int64_t n, int blocksize, const PreparedTable& t,
                    void* absmax, uint8_t* packed, bool nested, void* stream);
// Workgroups of a quantize launch over n elements.
int quantize_grid(int64_t n);
constexpr int64_t kQuantTileElems = 8192;  // elements per quantize tile
// Blocks per run of the nested mean's first level: each run is an aligned subtree of the
// pairwise tree, summed by one workgroup into one binary64 run sum.
constexpr int64_t kRunBlocks = 16384;
int launch_dequantize(void* out, int dtype, int64_t n, int blocksize, const DequantArgs& a,
                      const float* absmax, const uint8_t* packed, void* stream);
// absmax: the block maxima as the nested data pass stores them for `dtype` (binary32 for fp32
// input, the 16-bit pattern for fp16 / bf16 input); runs: ceil(nb / kRunBlocks) binary64 run
// sums (workspace).
int launch_nested_stats(const void* absmax, int dtype, int64_t nb, int blocksize2, const PreparedTable& t2,
                        double* runs, uint8_t* q2, float* absmax2, float* mean, void* stream);
int launch_dequantize_nested(void* out, int dtype, int64_t n, int blocksize, int blocksize2,
                             const NestedDequantArgs& a, const uint8_t* q2, const float* absmax2,
                             const float* mean, const uint8_t* packed, void* stream);
int launch_q32(const void* blocks, int dtype, int64_t n, int fmt, void* out, void* stream);
int launch_iq2xs_quantize(const void* in, int dtype, int64_t n, const uint8_t* grid, const uint16_t* scales,
                          uint8_t* blocks, uint32_t* rejected, void* stream);
int launch_iq2xs_dequantize(const uint8_t* blocks, const uint8_t* grid, int64_t n, int dtype, void* out,
                            void* stream);
int launch_iq1s_quantize(const void* in, int dtype, int64_t n, const int8_t* grid, uint8_t* blocks, void* stream);
int launch_iq1s_dequantize(const uint8_t* blocks, const int8_t* grid, int64_t n, int dtype, void* out,
                           void* stream);

// The library-owned scratch of bq_quantize_nested_noalloc (k_scratch.hip): kScratchBytes per
// device, 256-byte aligned.  scratch_buffer sets *ptr to the current device's copy (its device
// address, looked up once per device) and returns 0, or a hipError_t.
constexpr size_t kScratchBytes = (size_t)36 << 20;
int scratch_buffer(void** ptr);
}  // namespace bq
