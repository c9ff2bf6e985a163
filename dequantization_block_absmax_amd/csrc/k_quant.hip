// k_quant.hip -- blockwise absmax quantization kernels for gfx950.
//
// Rules (the blockwise family of "Respect the current CUDA stream in blockwise
// quantization", bitsandbytes PR 2052, Summary and "Correctness and safety"):
//   a_b = max |x_i| over the finite x_i of block b (+0 if none);
//   y_i = fl32(fl32(x_i * s) * fl32(1 / fl32(a_b * s))), s the power-of-two guard;
//   q_i = nearest code, ties to the lower index; non-finite x_i and zero blocks -> z;
//   4-bit: two codes per byte, first element in the high nibble, zero pad nibble.
//
// Work decomposition.  A lane owns 32 consecutive elements (64 B of bf16/fp16, 128 B of
// fp32), loaded with 16-byte vector loads; its 4-bit codes are one 16-byte store, so the
// stores of consecutive lanes are contiguous.  A block of B elements is G = B/32 consecutive
// lanes: G <= 64 reduce the absmax within the wave by xor-shuffles, G = 128 (B = 4096) adds
// one LDS exchange between the two waves.  A 256-lane workgroup covers 8192 elements per
// tile and `tiles` consecutive tiles; the grid is not persistent.
//
// The absmax uses an integer key: k = (bits << 1) + OFF (mod 2^w) drops the sign and wraps
// NaN/Inf below every finite value, so max(k) excludes non-finite elements without a compare.
#include <hip/hip_runtime.h>

#include "bq_device.h"
#include "bq_launch.h"

namespace bq {
namespace {

constexpr int kThreads = 256;
constexpr int kEPT = 32;
constexpr int kTile = kThreads * kEPT;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <int DT>
struct Traits {
  static constexpr int kWords = DT == F32 ? 32 : 16;  // 32-bit words per lane chunk
  static constexpr uint32_t kNaNWord = DT == F32 ? 0x7fc00000u : DT == BF16 ? 0x7fc07fc0u : 0x7e007e00u;
};

// Element e of the lane chunk, widened exactly to binary32.
template <int DT>
__device__ __forceinline__ float widen(const uint32_t* w, int e) {
  if constexpr (DT == F32) {
    return bits_f32(w[e]);
  } else if constexpr (DT == BF16) {
    uint32_t v = w[e >> 1];
    return bits_f32((e & 1) ? (v & 0xffff0000u) : (v << 16));
  } else {
    uint32_t v = w[e >> 1];
    unsigned short h = (unsigned short)((e & 1) ? (v >> 16) : (v & 0xffffu));
    return (float)__builtin_bit_cast(_Float16, h);
  }
}

// Max of the finite-|x| key over the lane chunk.
template <int DT>
__device__ __forceinline__ uint32_t chunk_key(const uint32_t* w) {
  if constexpr (DT == F32) {
    uint32_t k = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) k = max(k, (w[i] << 1) + 0x01000000u);
    return k;
  } else {
    constexpr unsigned short off = DT == BF16 ? 0x0100 : 0x0800;
    u16x2 acc = {0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      u16x2 h = __builtin_bit_cast(u16x2, w[i]);
      u16x2 k = (h << (unsigned short)1) + (u16x2){off, off};
      acc = __builtin_elementwise_max(acc, k);
    }
    return max((uint32_t)acc.x, (uint32_t)acc.y);
  }
}

// Block absmax (binary32) from the max key; +0 when the block has no finite element.
template <int DT>
__device__ __forceinline__ float key_to_absmax(uint32_t k) {
  if constexpr (DT == F32) {
    return bits_f32(k >= 0x01000000u ? (k - 0x01000000u) >> 1 : 0u);
  } else if constexpr (DT == BF16) {
    return bits_f32((k >= 0x0100u ? (k - 0x0100u) >> 1 : 0u) << 16);
  } else {
    unsigned short h = (unsigned short)(k >= 0x0800u ? (k - 0x0800u) >> 1 : 0u);
    return (float)__builtin_bit_cast(_Float16, h);
  }
}

template <int DT, int KB, int MODE, int M>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const uint8_t* __restrict__ in, int64_t n,
                                                            int log2g, int tiles,
                                                            float* __restrict__ absmax,
                                                            uint8_t* __restrict__ packed, QuantArgs qa) {
  using Tr = Traits<DT>;
  using E = typename Entry<M>::type;
  __shared__ float s_thr[260];
  __shared__ E s_lut[MODE == SEARCH ? 1 : kLutMax];
  __shared__ uint32_t s_red[kThreads / 64];

  const int tid = threadIdx.x;
  build_lut<MODE, M>(qa, s_lut, s_thr, tid, kThreads);

  const int G = 1 << log2g;
  const int B = kEPT << log2g;
  const int64_t nb = (n + B - 1) / B;
  const int64_t packed_bytes = KB == 4 ? (n + 1) / 2 : n;
  const int lane = tid & 63;

  for (int t = 0; t < tiles; ++t) {
    const int64_t elem0 = ((int64_t)(blockIdx.x * tiles + t) * kThreads + tid) * kEPT;
    uint32_t w[Tr::kWords];
    int nvalid = 32;
    if (elem0 + kEPT <= n) {
      const uint4* src = reinterpret_cast<const uint4*>(in + elem0 * (DT == F32 ? 4 : 2));
#pragma unroll
      for (int i = 0; i < Tr::kWords / 4; ++i) {
        uint4 v = src[i];
        w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
      }
    } else {
      nvalid = elem0 < n ? (int)(n - elem0) : 0;
#pragma unroll
      for (int i = 0; i < Tr::kWords; ++i) w[i] = Tr::kNaNWord;  // NaN pads: excluded from absmax
      if constexpr (DT == F32) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(in) + elem0;
#pragma unroll
        for (int e = 0; e < 32; ++e)
          if (e < nvalid) w[e] = src[e];
      } else {
        const unsigned short* src = reinterpret_cast<const unsigned short*>(in) + elem0;
#pragma unroll
        for (int e = 0; e < 32; ++e)
          if (e < nvalid)
            w[e >> 1] = (e & 1) ? ((w[e >> 1] & 0xffffu) | ((uint32_t)src[e] << 16))
                                : ((w[e >> 1] & 0xffff0000u) | src[e]);
      }
    }

    // Block absmax over G lanes.
    uint32_t key = chunk_key<DT>(w);
    for (int m = 1; m < G && m < 64; m <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, m));
    if (G > 64) {  // B = 4096: two waves per block
      if (lane == 0) s_red[tid >> 6] = key;
      __syncthreads();
      key = max(s_red[tid >> 6], s_red[(tid >> 6) ^ 1]);
      __syncthreads();
    }
    const float a = key_to_absmax<DT>(key);
    const int64_t blk = elem0 >> (5 + log2g);
    if ((tid & (G - 1)) == 0 && blk < nb) absmax[blk] = a;

    // Normalize with the power-of-two guard.
    const float s = a < 0x1p-64f ? 0x1p64f : (a > 0x1p64f ? 0x1p-64f : 1.0f);
    const float r = 1.0f / (a * s);
    uint32_t q[32];
    if (s == 1.0f) {
#pragma unroll
      for (int e = 0; e < 32; ++e) q[e] = nearest_code<MODE, M>(widen<DT>(w, e) * r, qa, s_lut, s_thr);
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) q[e] = nearest_code<MODE, M>((widen<DT>(w, e) * s) * r, qa, s_lut, s_thr);
    }
    if (nvalid < 32) {
#pragma unroll
      for (int e = 0; e < 32; ++e) q[e] = e < nvalid ? q[e] : 0u;  // zero pad nibble / unused codes
    }

    // Pack and store.
    if constexpr (KB == 4) {
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) v |= ((q[8 * i + 2 * b] << 4) | q[8 * i + 2 * b + 1]) << (8 * b);
        o[i] = v;
      }
      const int64_t off = elem0 >> 1;
      if (off + 16 <= packed_bytes) {
        *reinterpret_cast<uint4*>(packed + off) = make_uint4(o[0], o[1], o[2], o[3]);
      } else if (off < packed_bytes) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (off + i < packed_bytes) packed[off + i] = (uint8_t)(o[i >> 2] >> (8 * (i & 3)));
      }
    } else {
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = q[4 * i] | (q[4 * i + 1] << 8) | (q[4 * i + 2] << 16) | (q[4 * i + 3] << 24);
      const int64_t off = elem0;
      if (off + 32 <= packed_bytes) {
        uint4* dst = reinterpret_cast<uint4*>(packed + off);
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
      } else if (off < packed_bytes) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if (off + i < packed_bytes) packed[off + i] = (uint8_t)(o[i >> 2] >> (8 * (i & 3)));
      }
    }
  }
}

template <int DT, int KB, int MODE, int M>
hipError_t launch4(const void* in, int64_t n, int log2g, float* absmax, uint8_t* packed, const QuantArgs& qa,
                   hipStream_t stream) {
  const int64_t tiles_total = (n + kTile - 1) / kTile;
  const int tiles = 1;
  const int64_t grid = (tiles_total + tiles - 1) / tiles;
  return launch_kernel(quantize_kernel<DT, KB, MODE, M>, dim3((unsigned)grid), dim3(kThreads), stream,
                       static_cast<const uint8_t*>(in), n, log2g, tiles, absmax, packed, qa);
}

template <int DT, int KB>
hipError_t launch_mode(const void* in, int64_t n, int log2g, float* absmax, uint8_t* packed,
                       const PreparedTable& t, hipStream_t s) {
  if (t.mode == LIN) {
    if (t.M <= 1) return launch4<DT, KB, LIN, 1>(in, n, log2g, absmax, packed, t.qa, s);
    if (t.M == 2) return launch4<DT, KB, LIN, 2>(in, n, log2g, absmax, packed, t.qa, s);
    return launch4<DT, KB, LIN, 3>(in, n, log2g, absmax, packed, t.qa, s);
  }
  if (t.mode == LOG) {
    if (t.M <= 1) return launch4<DT, KB, LOG, 1>(in, n, log2g, absmax, packed, t.qa, s);
    if (t.M == 2) return launch4<DT, KB, LOG, 2>(in, n, log2g, absmax, packed, t.qa, s);
    return launch4<DT, KB, LOG, 3>(in, n, log2g, absmax, packed, t.qa, s);
  }
  return launch4<DT, KB, SEARCH, 1>(in, n, log2g, absmax, packed, t.qa, s);
}

template <int DT>
hipError_t launch_dt(const void* in, int64_t n, int log2g, float* absmax, uint8_t* packed, const PreparedTable& t,
                     hipStream_t s) {
  return t.K == 16 ? launch_mode<DT, 4>(in, n, log2g, absmax, packed, t, s)
                   : launch_mode<DT, 8>(in, n, log2g, absmax, packed, t, s);
}

}  // namespace

int launch_quantize(const void* in, int dtype, int64_t n, int blocksize, const PreparedTable& t, float* absmax,
                    uint8_t* packed, void* stream) {
  int log2g = 0;
  while ((kEPT << log2g) < blocksize) ++log2g;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == F32) e = launch_dt<F32>(in, n, log2g, absmax, packed, t, s);
  else if (dtype == F16) e = launch_dt<F16>(in, n, log2g, absmax, packed, t, s);
  else e = launch_dt<BF16>(in, n, log2g, absmax, packed, t, s);
  return (int)e;
}

}  // namespace bq
