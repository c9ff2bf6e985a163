// k_dequant.hip -- blockwise dequantization kernels for gfx950.
//
//   out_i = RN(fl32(c[q_i] * a_b))            blockwise
//   a'_b  = fl32(fl32(c2[q2_b] * a2_g) + mean) nested statistics, then as above
// (the inverse of the blockwise quantization of "Respect the current CUDA stream in blockwise
// quantization", bitsandbytes PR 2052; nested statistics from its "Reproduced failure").
//
// Work decomposition.  A unit is 8 consecutive elements: 4 bytes of 4-bit codes or 8 bytes of
// 8-bit codes in, 16 bytes of bf16/fp16 (32 of fp32) out.  Lane `tid` of a 256-lane
// workgroup handles units tile*1024 + u*256 + tid for u = 0..3, so every load and store
// instruction of a wave touches one contiguous span (per-lane contiguous 64-byte writes
// measured at half the bandwidth of this layout on MI355X).  The table lives in LDS; the
// binary32 product is rounded once by the hardware conversion (round-to-nearest-even).
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "bq_launch.h"

namespace bq {
namespace {

constexpr int kThreads = 256;
constexpr int kUnits = 4;                          // units per lane per workgroup
constexpr int kTileElems = kThreads * kUnits * 8;  // 8192

// Stores 8 binary32 values as `DT` at element offset e (full unit).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Non-temporal 16-byte store: output streams straight to memory (measured on MI355X at
// ~89% of HBM peak for a 1:4 read:write stream, against ~74% with ordinary stores).
__device__ __forceinline__ void store16_nt(uint8_t* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

template <int DT>
__device__ __forceinline__ void store8(uint8_t* out, int64_t e, const float* v) {
  if constexpr (DT == F32) {
    uint8_t* dst = out + e * 4;
    store16_nt(dst, f32_bits(v[0]), f32_bits(v[1]), f32_bits(v[2]), f32_bits(v[3]));
    store16_nt(dst + 16, f32_bits(v[4]), f32_bits(v[5]), f32_bits(v[6]), f32_bits(v[7]));
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t lo, hi;
      if constexpr (DT == BF16) {
        lo = __builtin_bit_cast(uint16_t, (__bf16)v[2 * i]);
        hi = __builtin_bit_cast(uint16_t, (__bf16)v[2 * i + 1]);
      } else {
        lo = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i]);
        hi = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1]);
      }
      w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    store16_nt(out + e * 2, w[0], w[1], w[2], w[3]);
  }
}

// Stores the first `cnt` (< 8) values of a tail unit one element at a time.
template <int DT>
__device__ __forceinline__ void store_tail(uint8_t* out, int64_t e, const float* v, int cnt) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < cnt) {
      if constexpr (DT == F32) reinterpret_cast<float*>(out)[e + i] = v[i];
      else if constexpr (DT == BF16) reinterpret_cast<__bf16*>(out)[e + i] = (__bf16)v[i];
      else reinterpret_cast<_Float16*>(out)[e + i] = (_Float16)v[i];
    }
  }
}

// Codes of a unit starting at element e (e a multiple of 8).
template <int KB>
__device__ __forceinline__ void load_codes(const uint8_t* packed, int64_t e, int64_t n, uint32_t* q) {
  if constexpr (KB == 4) {
    uint32_t p;
    if (e + 8 <= n) {
      p = *reinterpret_cast<const uint32_t*>(packed + (e >> 1));
    } else {
      p = 0;
      const int64_t nbytes = (n + 1) >> 1;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((e >> 1) + i < nbytes) p |= (uint32_t)packed[(e >> 1) + i] << (8 * i);
    }
    // byte b holds element 2b in its high nibble and element 2b+1 in its low nibble
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      q[2 * b] = (p >> (8 * b + 4)) & 15u;
      q[2 * b + 1] = (p >> (8 * b)) & 15u;
    }
  } else {
    uint2 p;
    if (e + 8 <= n) {
      p = *reinterpret_cast<const uint2*>(packed + e);
    } else {
      p = make_uint2(0, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (e + i < n) {
          uint32_t byte = packed[e + i];
          if (i < 4) p.x |= byte << (8 * i);
          else p.y |= byte << (8 * (i - 4));
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[i] = (p.x >> (8 * i)) & 255u;
      q[4 + i] = (p.y >> (8 * i)) & 255u;
    }
  }
}

// A lane takes its units one after another (load, scale, store).  Issuing all of a lane's
// loads first measured slower on MI355X for the nested kernel (314 us against 273 us on
// 2^29 bf16 outputs), and no faster for the plain one.
template <int DT, int KB>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const uint8_t* __restrict__ packed,
                                                              const float* __restrict__ absmax, int64_t n,
                                                              int log2b, uint8_t* __restrict__ out,
                                                              DequantArgs da) {
  __shared__ float s_c[256];
  const int tid = threadIdx.x;
  s_c[tid] = tid < da.K ? da.c[tid] : 0.0f;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    const int64_t e = (((int64_t)blockIdx.x * kUnits + u) * kThreads + tid) * 8;
    if (e >= n) break;
    uint32_t q[8];
    load_codes<KB>(packed, e, n, q);
    const float a = absmax[e >> log2b];
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = s_c[q[i]] * a;
    if (e + 8 <= n) store8<DT>(out, e, v);
    else store_tail<DT>(out, e, v, (int)(n - e));
  }
}

template <int DT, int KB>
__global__ __launch_bounds__(kThreads) void dequantize_nested_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ q2, const float* __restrict__ absmax2,
    const float* __restrict__ mean, int64_t n, int log2b, int log2b2, uint8_t* __restrict__ out,
    NestedDequantArgs da) {
  __shared__ float s_c[256];
  __shared__ float s_c2[256];
  const int tid = threadIdx.x;
  s_c[tid] = tid < da.K ? da.c[tid] : 0.0f;
  s_c2[tid] = da.c2[tid];
  const float m = *mean;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    const int64_t e = (((int64_t)blockIdx.x * kUnits + u) * kThreads + tid) * 8;
    if (e >= n) break;
    uint32_t q[8];
    load_codes<KB>(packed, e, n, q);
    const int64_t b = e >> log2b;
    const float scaled = s_c2[q2[b]] * absmax2[b >> log2b2];
    const float a = scaled + m;  // two roundings, no fused multiply-add
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = s_c[q[i]] * a;
    if (e + 8 <= n) store8<DT>(out, e, v);
    else store_tail<DT>(out, e, v, (int)(n - e));
  }
}

int ilog2(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

template <int KB>
hipError_t launch_dq(void* out, int dtype, int64_t n, int blocksize, const DequantArgs& a, const float* absmax,
                     const uint8_t* packed, hipStream_t s) {
  const unsigned grid = (unsigned)((n + kTileElems - 1) / kTileElems);
  const int lb = ilog2(blocksize);
  uint8_t* o = static_cast<uint8_t*>(out);
  if (dtype == F32)
    return launch_kernel(dequantize_kernel<F32, KB>, dim3(grid), dim3(kThreads), s, packed, absmax, n, lb, o, a);
  if (dtype == F16)
    return launch_kernel(dequantize_kernel<F16, KB>, dim3(grid), dim3(kThreads), s, packed, absmax, n, lb, o, a);
  return launch_kernel(dequantize_kernel<BF16, KB>, dim3(grid), dim3(kThreads), s, packed, absmax, n, lb, o, a);
}

template <int KB>
hipError_t launch_dqn(void* out, int dtype, int64_t n, int blocksize, int blocksize2, const NestedDequantArgs& a,
                      const uint8_t* q2, const float* absmax2, const float* mean, const uint8_t* packed,
                      hipStream_t s) {
  const unsigned grid = (unsigned)((n + kTileElems - 1) / kTileElems);
  const int lb = ilog2(blocksize), lb2 = ilog2(blocksize2);
  uint8_t* o = static_cast<uint8_t*>(out);
  if (dtype == F32)
    return launch_kernel(dequantize_nested_kernel<F32, KB>, dim3(grid), dim3(kThreads), s, packed, q2, absmax2,
                         mean, n, lb, lb2, o, a);
  if (dtype == F16)
    return launch_kernel(dequantize_nested_kernel<F16, KB>, dim3(grid), dim3(kThreads), s, packed, q2, absmax2,
                         mean, n, lb, lb2, o, a);
  return launch_kernel(dequantize_nested_kernel<BF16, KB>, dim3(grid), dim3(kThreads), s, packed, q2, absmax2,
                       mean, n, lb, lb2, o, a);
}

}  // namespace

int launch_dequantize(void* out, int dtype, int64_t n, int blocksize, const DequantArgs& a, const float* absmax,
                      const uint8_t* packed, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return (int)(a.K == 16 ? launch_dq<4>(out, dtype, n, blocksize, a, absmax, packed, s)
                         : launch_dq<8>(out, dtype, n, blocksize, a, absmax, packed, s));
}

int launch_dequantize_nested(void* out, int dtype, int64_t n, int blocksize, int blocksize2,
                             const NestedDequantArgs& a, const uint8_t* q2, const float* absmax2,
                             const float* mean, const uint8_t* packed, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return (int)(a.K == 16 ? launch_dqn<4>(out, dtype, n, blocksize, blocksize2, a, q2, absmax2, mean, packed, s)
                         : launch_dqn<8>(out, dtype, n, blocksize, blocksize2, a, q2, absmax2, mean, packed, s));
}

}  // namespace bq
