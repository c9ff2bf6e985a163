// k_q32.hip -- dequantization of GGUF-style 32-element blocks (the Q4_0 / Q8_0 shapes of
// "Cache device-side constants in dequant kernels", ComfyUI-GGUF PR 472, "Verification").
//
//   Q4 block (18 B): binary16 d, then 16 bytes; element j < 16 = low nibble of byte j,
//                    element 16 + j = high nibble of byte j (low nibbles of a group precede
//                    its high nibbles, the shift-by-{0,4} idiom of that page's "Problem");
//                    value = RN(fl32((q - 8) * d)).
//   Q8 block (34 B): binary16 d, then 32 int8; value = RN(fl32(q * d)).
// The binary32 products are exact (at most 5 x 11 or 8 x 11 significant bits), so each
// output is rounded exactly once, by the conversion to the output type.
//
// Work decomposition: a unit is a quarter block (8 elements, 16 output bytes for bf16).
// Lane `tid` of a 256-lane workgroup handles units tile*1024 + u*256 + tid, u = 0..3, so the
// output stores of a wave are contiguous.  Blocks are only 2-byte aligned (18 and 34 bytes),
// so the 8 payload bytes of a unit are read as 16-bit loads.
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "bq_launch.h"

namespace bq {
namespace {

constexpr int kThreads = 256;
constexpr int kUnits = 4;

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

template <int DT, int FMT>
__global__ __launch_bounds__(kThreads) void q32_kernel(const uint8_t* __restrict__ blocks, int64_t n,
                                                       uint8_t* __restrict__ out) {
  constexpr int BS = FMT == 0 ? 18 : 34;
  const int tid = threadIdx.x;
  // All loads of the lane's units first (n is a multiple of 32: units are whole).
  int64_t unit[kUnits];
  uint16_t dbits[kUnits];
  uint32_t lo[kUnits], hi[kUnits];
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    unit[u] = ((int64_t)blockIdx.x * kUnits + u) * kThreads + tid;
    if (unit[u] * 8 < n) {
      const int k = (int)(unit[u] & 3);
      const uint8_t* bp = blocks + (unit[u] >> 2) * BS;
      dbits[u] = *reinterpret_cast<const uint16_t*>(bp);
      const uint16_t* pay = reinterpret_cast<const uint16_t*>(bp + 2 + (FMT == 0 ? 8 * (k & 1) : 8 * k));
      lo[u] = (uint32_t)pay[0] | ((uint32_t)pay[1] << 16);
      hi[u] = (uint32_t)pay[2] | ((uint32_t)pay[3] << 16);
    }
  }
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    if (unit[u] * 8 < n) {
      const int k = (int)(unit[u] & 3);
      const float d = (float)__builtin_bit_cast(_Float16, dbits[u]);
      float v[8];
      if constexpr (FMT == 0) {
        const int sh = (k & 2) ? 4 : 0;  // units 0,1: low nibbles; units 2,3: high nibbles
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = (float)((int)((lo[u] >> (8 * i + sh)) & 15u) - 8) * d;
          v[4 + i] = (float)((int)((hi[u] >> (8 * i + sh)) & 15u) - 8) * d;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = (float)(int)(int8_t)(lo[u] >> (8 * i)) * d;
          v[4 + i] = (float)(int)(int8_t)(hi[u] >> (8 * i)) * d;
        }
      }
      store8<DT>(out, unit[u] * 8, v);
    }
  }
}

template <int FMT>
hipError_t launch_fmt(const void* blocks, int dtype, int64_t n, void* out, hipStream_t s) {
  const unsigned grid = (unsigned)((n / 8 + kThreads * kUnits - 1) / (kThreads * kUnits));
  const uint8_t* b = static_cast<const uint8_t*>(blocks);
  uint8_t* o = static_cast<uint8_t*>(out);
  if (dtype == F32) return launch_kernel(q32_kernel<F32, FMT>, dim3(grid), dim3(kThreads), s, b, n, o);
  if (dtype == F16) return launch_kernel(q32_kernel<F16, FMT>, dim3(grid), dim3(kThreads), s, b, n, o);
  return launch_kernel(q32_kernel<BF16, FMT>, dim3(grid), dim3(kThreads), s, b, n, o);
}

}  // namespace

int launch_q32(const void* blocks, int dtype, int64_t n, int fmt, void* out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return (int)(fmt == 0 ? launch_fmt<0>(blocks, dtype, n, out, s) : launch_fmt<1>(blocks, dtype, n, out, s));
}

}  // namespace bq
