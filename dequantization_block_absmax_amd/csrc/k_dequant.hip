// k_dequant.hip -- blockwise dequantization kernels for gfx950.
//
//   out_i = RN(fl32(c[q_i] * a_b))            blockwise
//   a'_b  = fl32(fl32(c2[q2_b] * a2_g) + mean) nested statistics, then as above
// (the inverse of the blockwise quantization of "Respect the current CUDA stream in blockwise
// quantization", bitsandbytes PR 2052; nested statistics from its "Reproduced failure").
//
// Work decomposition.  A unit is 8 consecutive elements: 4 bytes of 4-bit codes or 8 bytes of
// 8-bit codes in, 16 bytes of bf16/fp16 (32 of fp32) out.  Lane `tid` of a 256-lane
// workgroup handles units tile*256*U + u*256 + tid for u < U (U = 4 for 4-bit codes, 2 for 8-bit), so
// every load and store instruction of a wave touches one contiguous span (per-lane
// contiguous 64-byte writes measured at half the bandwidth of this layout on MI355X).  The
// tile's block scales are staged in LDS while the lane's code loads are in flight.
// The table lives in LDS; the binary32 product is rounded once by the hardware conversion
// (round-to-nearest-even).
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "bq_launch.h"

namespace bq {
namespace {

constexpr int kThreads = 256;
// Units per lane: 4 for 4-bit codes (a 8192-element tile), 2 for 8-bit codes (4096), the
// faster of 2, 4 and 8 for each on MI355X.
template <int KB>
struct Tile {
  static constexpr int kUnits = KB == 4 ? 4 : 2;
  static constexpr int kElems = kThreads * kUnits * 8;
  static constexpr int kBlocks = kElems / 32;  // most blocks a tile can touch (B >= 32)
};

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

// Raw code bytes of the unit starting at element e (e a multiple of 8, e < n): 4 bytes of
// nibbles (4-bit) or 8 code bytes (8-bit); bytes past the end of `packed` read as 0.
// In the tail unit each byte is loaded into its own register and the words are joined after
// by byte permutes, so the loads are in flight together (merging each byte into its word as it
// arrives made every load wait for the previous one).
__device__ __forceinline__ uint32_t join_bytes(const uint32_t* b) {
  return __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                               __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u), 0x05040100u);
}

template <int KB>
__device__ __forceinline__ uint2 fetch_codes(const uint8_t* packed, int64_t e, int64_t n) {
  uint2 p = make_uint2(0, 0);
  if constexpr (KB == 4) {
    if (e + 8 <= n) {
      p.x = *reinterpret_cast<const uint32_t*>(packed + (e >> 1));
    } else {
      const int64_t nbytes = (n + 1) >> 1;
      uint32_t b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = (e >> 1) + i < nbytes ? (uint32_t)packed[(e >> 1) + i] : 0u;
      p.x = join_bytes(b);
    }
  } else {
    if (e + 8 <= n) {
      p = *reinterpret_cast<const uint2*>(packed + e);
    } else {
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = e + i < n ? (uint32_t)packed[e + i] : 0u;
      p.x = join_bytes(b);
      p.y = join_bytes(b + 4);
    }
  }
  return p;
}

// The 8 codes of a unit from its raw bytes.
template <int KB>
__device__ __forceinline__ void decode_codes(uint2 p, uint32_t* q) {
  if constexpr (KB == 4) {
    // byte b holds element 2b in its high nibble and element 2b+1 in its low nibble
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      q[2 * b] = (p.x >> (8 * b + 4)) & 15u;
      q[2 * b + 1] = (p.x >> (8 * b)) & 15u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[i] = (p.x >> (8 * i)) & 255u;
      q[4 + i] = (p.y >> (8 * i)) & 255u;
    }
  }
}

// Block scales of a tile are staged in LDS, each block's by one thread: one coalesced load
// per block instead of one gather per unit.  With per-unit gathers of the nested statistics the kernel ran at 62% of HBM
// peak on 2^29 bf16 outputs, against 90% without them.

// Blocks of the tile starting at element e0: [e0 >> log2b, last element's block].
template <int KB>
__device__ __forceinline__ int tile_blocks(int64_t e0, int64_t n, int log2b) {
  const int64_t e1 = min(e0 + (int64_t)Tile<KB>::kElems, n) - 1;
  return (int)((e1 >> log2b) - (e0 >> log2b)) + 1;
}

// A lane's code loads, issued before the workgroup prologue so that they overlap it.  FULL:
// the tile lies inside [0, n), and every load is unconditional.  8-bit codes load
// non-temporally (bf16 2^26, B = 4096: 31.6 against 32.9 us); for 4-bit codes the hint measured
// slower (2^29 nested: 210.7 against 205.9 us).
template <int KB, bool FULL>
__device__ __forceinline__ void fetch_tile(const uint8_t* __restrict__ packed, int64_t n, int64_t e0, uint2* raw) {
#pragma unroll
  for (int u = 0; u < Tile<KB>::kUnits; ++u) {
    const int64_t e = e0 + (int64_t)(u * kThreads + threadIdx.x) * 8;
    if constexpr (FULL) {
      typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));
      if constexpr (KB == 4) {
        raw[u] = make_uint2(*reinterpret_cast<const uint32_t*>(packed + (e >> 1)), 0u);
      } else {
        const u32x2_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(packed + e));
        raw[u] = make_uint2(v.x, v.y);
      }
    } else {
      raw[u] = e < n ? fetch_codes<KB>(packed, e, n) : make_uint2(0, 0);
    }
  }
}

// Scales and stores the lane's units.
template <int DT, int KB, bool FULL>
__device__ __forceinline__ void emit_tile(const uint2* raw, int64_t n, int log2b, int64_t e0, const float* s_c,
                                          const float* s_a, uint8_t* __restrict__ out) {
  const int64_t b0 = e0 >> log2b;
#pragma unroll
  for (int u = 0; u < Tile<KB>::kUnits; ++u) {
    const int64_t e = e0 + (int64_t)(u * kThreads + threadIdx.x) * 8;
    if (!FULL && e >= n) break;
    uint32_t q[8];
    decode_codes<KB>(raw[u], q);
    const float a = s_a[(int)((e >> log2b) - b0)];
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = s_c[q[i]] * a;
      // The binary32 product is rounded before the conversion: fused into one mixed-precision
      // fma (v_fma_mixlo_f16) it would round once, and differ where rounding twice does not
      // give the same half-precision value.
      if constexpr (DT == F16) asm("" : "+v"(v[i]));
    }
    if (FULL || e + 8 <= n) store8<DT>(out, e, v);
    else store_tail<DT>(out, e, v, (int)(n - e));
  }
}

// Workgroup barrier for data exchanged through LDS only: it waits for this wave's LDS
// accesses, not for its outstanding global loads (the tile's codes stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The tile's block scales are staged in LDS, each block's by one thread (a tile spans at most
// 256 blocks).  Two orders, each the faster on MI355X for its code width (interleaved A/B):
// - 8-bit codes: the scale and table loads are issued first and with no condition around
//   them, then the code loads; the LDS staging then waits for the scales only, and the
//   codes stay in flight.  (Where a load under a condition joins a path without it, the
//   compiler can only wait for every outstanding load, so threads past the tile's blocks load
//   and store the last block's scale into a slot that is never read.)  bf16 2^26, B = 4096:
//   32.9 µs against 35.0 for the other order and 37.0 for per-unit conditional code loads.
// - 4-bit codes, whose output is four times their input: the code loads first, then the
//   scales under a condition, and the workgroup waits for all of them before it stores, in
//   one burst.  bf16 2^29, B = 64: 225.3 µs against 229.5 for the 8-bit order.
template <int DT, int KB, bool FULL>
__device__ __forceinline__ void dequant_tile(const uint8_t* __restrict__ packed, const float* __restrict__ absmax,
                                             int64_t n, int log2b, uint8_t* __restrict__ out, const DequantArgs& da,
                                             int64_t e0, float* s_c, float* s_a) {
  const int tid = threadIdx.x;
  const int nblk = tile_blocks<KB>(e0, n, log2b);
  uint2 raw[Tile<KB>::kUnits];
  if constexpr (KB == 8) {
    const float c = da.c[tid];  // entries past K are zero
    const float a = absmax[(e0 >> log2b) + min(tid, nblk - 1)];
    fetch_tile<KB, FULL>(packed, n, e0, raw);
    s_c[tid] = c;
    s_a[tid] = a;
    lds_barrier();
  } else {
    fetch_tile<KB, FULL>(packed, n, e0, raw);
    s_c[tid] = da.c[tid];
    if (tid < nblk) s_a[tid] = absmax[(e0 >> log2b) + tid];
    __syncthreads();
  }
  emit_tile<DT, KB, FULL>(raw, n, log2b, e0, s_c, s_a, out);
}

template <int DT, int KB>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const uint8_t* __restrict__ packed,
                                                              const float* __restrict__ absmax, int64_t n,
                                                              int log2b, uint8_t* __restrict__ out,
                                                              DequantArgs da) {
  static_assert(Tile<KB>::kBlocks <= kThreads, "one thread per block of a tile");
  __shared__ float s_c[256];
  __shared__ float s_a[kThreads];
  const int64_t e0 = (int64_t)blockIdx.x * Tile<KB>::kElems;
  if (e0 + Tile<KB>::kElems <= n) dequant_tile<DT, KB, true>(packed, absmax, n, log2b, out, da, e0, s_c, s_a);
  else dequant_tile<DT, KB, false>(packed, absmax, n, log2b, out, da, e0, s_c, s_a);
}

// As dequant_tile, with the scale a'_b = fl32(fl32(c2[q2_b] * a2_g) + mean) built from the
// nested statistics by one thread per block once the second table is in LDS.  The code loads
// come first and the workgroup waits for all loads before it stores (bf16 2^29 4-bit, B = 64,
// groups of 256: 200.3 µs, against 215.3 with the statistics loads issued first and 204.3
// with per-unit conditional code loads).
template <int DT, int KB, bool FULL>
__device__ __forceinline__ void dequant_nested_tile(const uint8_t* __restrict__ packed,
                                                    const uint8_t* __restrict__ q2,
                                                    const float* __restrict__ absmax2, const float* __restrict__ mean,
                                                    int64_t n, int log2b, int log2b2, uint8_t* __restrict__ out,
                                                    const NestedDequantArgs& da, int64_t e0, float* s_c,
                                                    float* s_c2, float* s_a) {
  const int tid = threadIdx.x;
  const int nblk = tile_blocks<KB>(e0, n, log2b);
  uint2 raw[Tile<KB>::kUnits];
  fetch_tile<KB, FULL>(packed, n, e0, raw);
  uint32_t code2 = 0;
  float a2 = 0.0f;
  if (tid < nblk) {
    const int64_t b = (e0 >> log2b) + tid;
    code2 = q2[b];
    a2 = absmax2[b >> log2b2];
  }
  s_c[tid] = da.c[tid];  // entries past K are zero
  s_c2[tid] = da.c2[tid];
  const float m = *mean;
  __syncthreads();
  if (tid < nblk) {
    const float scaled = s_c2[code2] * a2;
    s_a[tid] = scaled + m;  // two roundings, no fused multiply-add
  }
  __syncthreads();
  emit_tile<DT, KB, FULL>(raw, n, log2b, e0, s_c, s_a, out);
}

template <int DT, int KB>
__global__ __launch_bounds__(kThreads) void dequantize_nested_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ q2, const float* __restrict__ absmax2,
    const float* __restrict__ mean, int64_t n, int log2b, int log2b2, uint8_t* __restrict__ out,
    NestedDequantArgs da) {
  static_assert(Tile<KB>::kBlocks <= kThreads, "one thread per block of a tile");
  __shared__ float s_c[256];
  __shared__ float s_c2[256];
  __shared__ float s_a[kThreads];
  const int64_t e0 = (int64_t)blockIdx.x * Tile<KB>::kElems;
  if (e0 + Tile<KB>::kElems <= n)
    dequant_nested_tile<DT, KB, true>(packed, q2, absmax2, mean, n, log2b, log2b2, out, da, e0, s_c, s_c2, s_a);
  else
    dequant_nested_tile<DT, KB, false>(packed, q2, absmax2, mean, n, log2b, log2b2, out, da, e0, s_c, s_c2, s_a);
}

int ilog2(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

template <int KB>
hipError_t launch_dq(void* out, int dtype, int64_t n, int blocksize, const DequantArgs& a, const float* absmax,
                     const uint8_t* packed, hipStream_t s) {
  const unsigned grid = (unsigned)((n + Tile<KB>::kElems - 1) / Tile<KB>::kElems);
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
  const unsigned grid = (unsigned)((n + Tile<KB>::kElems - 1) / Tile<KB>::kElems);
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
