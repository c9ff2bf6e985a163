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
// Lane `tid` of a 256-lane workgroup handles units tile*512 + u*256 + tid, u = 0..1, so the
// output stores of a wave are contiguous.  Blocks are only 2-byte aligned (18 and 34 bytes);
// a tile's bytes are staged through LDS with 16-byte loads.
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "bq_launch.h"

namespace bq {
namespace {

constexpr int kThreads = 256;
constexpr int kUnits = 2;  // 128 blocks per workgroup: 2.5% faster than 256, far faster than 64

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
        // The product is held in a register before the conversion: folded into it, the multiply
        // becomes a mixed-precision fma (v_fma_mixlo_f16) with a +0 addend, which turns the -0
        // of (q - 8) * d = 0 * (negative d) into +0.
        float a = v[2 * i], b = v[2 * i + 1];
        asm("" : "+v"(a), "+v"(b));
        lo = __builtin_bit_cast(uint16_t, (_Float16)a);
        hi = __builtin_bit_cast(uint16_t, (_Float16)b);
      }
      w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    store16_nt(out + e * 2, w[0], w[1], w[2], w[3]);
  }
}

// The 8 values of a unit (quarter block k) from its fp16 scale bits and 8 payload bytes.
template <int FMT>
__device__ __forceinline__ void unit_values(uint16_t dbits, uint32_t lo, uint32_t hi, int k, float* v) {
  const float d = (float)__builtin_bit_cast(_Float16, dbits);
  if constexpr (FMT == 0) {
    const int sh = (k & 2) ? 4 : 0;  // units 0,1: low nibbles; units 2,3: high nibbles
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = (float)((int)((lo >> (8 * i + sh)) & 15u) - 8) * d;
      v[4 + i] = (float)((int)((hi >> (8 * i + sh)) & 15u) - 8) * d;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = (float)(int)(int8_t)(lo >> (8 * i)) * d;
      v[4 + i] = (float)(int)(int8_t)(hi >> (8 * i)) * d;
    }
  }
}

// Payload byte offset of unit k inside its block (after the 2-byte scale).
template <int FMT>
__device__ __forceinline__ int unit_offset(int k) {
  return 2 + (FMT == 0 ? 8 * (k & 1) : 8 * k);
}

// A workgroup expands 128 blocks (4096 values).  When the tile is whole and the blocks are
// 16-byte aligned, the tile's 2304 (Q4) or 4352 (Q8) bytes are read as contiguous 16-byte
// chunks (non-temporal) into LDS, and every unit reads its scale and payload there: one
// global load per 16 bytes instead of five 2-byte loads per unit (the records are only 2-byte
// aligned).  Otherwise each unit reads its bytes from memory with 2-byte loads.
template <int DT, int FMT>
__global__ __launch_bounds__(kThreads) void q32_kernel(const uint8_t* __restrict__ blocks, int64_t n,
                                                       uint8_t* __restrict__ out) {
  constexpr int BS = FMT == 0 ? 18 : 34;
  constexpr int kTileBlocks = kThreads * kUnits / 4;
  constexpr int kChunks = kTileBlocks * BS / 16;
  constexpr int kPer = (kChunks + kThreads - 1) / kThreads;
  __shared__ uint4 s_raw[kChunks];
  const int tid = threadIdx.x;
  const int64_t blk0 = (int64_t)blockIdx.x * kTileBlocks;
  const bool staged = blk0 + kTileBlocks <= n / 32 && (reinterpret_cast<uintptr_t>(blocks) & 15) == 0;
  if (staged) {  // uniform
    const u32x4* src = reinterpret_cast<const u32x4*>(blocks + blk0 * BS);
    u32x4 t[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * kThreads;
      if (c < kChunks) t[i] = __builtin_nontemporal_load(src + c);
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * kThreads;
      if (c < kChunks) s_raw[c] = make_uint4(t[i].x, t[i].y, t[i].z, t[i].w);
    }
    __syncthreads();
    const uint16_t* raw = reinterpret_cast<const uint16_t*>(s_raw);
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int uu = u * kThreads + tid;  // unit in the tile
      const int k = uu & 3;
      const int h = (uu >> 2) * (BS / 2);  // the block's first halfword
      const int p = h + unit_offset<FMT>(k) / 2;
      const uint32_t lo = (uint32_t)raw[p] | ((uint32_t)raw[p + 1] << 16);
      const uint32_t hi = (uint32_t)raw[p + 2] | ((uint32_t)raw[p + 3] << 16);
      float v[8];
      unit_values<FMT>(raw[h], lo, hi, k, v);
      store8<DT>(out, ((int64_t)blockIdx.x * kUnits * kThreads + uu) * 8, v);
    }
    return;
  }
  // n is a multiple of 32: units are whole.
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    const int64_t unit = ((int64_t)blockIdx.x * kUnits + u) * kThreads + tid;
    if (unit * 8 >= n) break;
    const int k = (int)(unit & 3);
    const uint8_t* bp = blocks + (unit >> 2) * BS;
    const uint16_t* pay = reinterpret_cast<const uint16_t*>(bp + unit_offset<FMT>(k));
    const uint32_t lo = (uint32_t)pay[0] | ((uint32_t)pay[1] << 16);
    const uint32_t hi = (uint32_t)pay[2] | ((uint32_t)pay[3] << 16);
    float v[8];
    unit_values<FMT>(*reinterpret_cast<const uint16_t*>(bp), lo, hi, k, v);
    store8<DT>(out, unit * 8, v);
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
