// k_iq2xs.hip -- IQ2_XS-style search encoding and decoding of 256-element superblocks
// ("[OMNIML-5899] Add CUDA kernels for IQ packing", Model-Optimizer PR 2448: the review items
// "Wire format", "Even-parity sign field" and "Search equivalence", and the round-3 "IQ2_XS
// grouping" item).  The byte layout and the search are stated in bq.h.
//
// Encoder: one 256-lane workgroup per superblock.  Lane (wave w, lane l) serves vector
// v = 8w + l / 8 and entry slice k = l % 8 (grid entries k, k + 8, ..., k + 504), so the eight
// slices of a vector are the eight lanes of one half-row and the two vectors of a group are
// the two halves of one 16-lane row: reductions over slices and the group sum are DPP moves.
// The grid sits in LDS as binary32 magnitudes with their squared norms (18 KB).
//   Pass 1: for each of its 64 entries a lane forms the corrected dot (fma chain, then the
//           parity correction) and keeps it in a register, and updates the 16 running minima
//           of the error over its entries, one per local scale (s and s*s are wave-uniform,
//           in scalar registers; fma(s, -2 dot, xn) equals fma(-2s, dot, xn) bit for bit, the
//           doubling being exact, so -2 dot is formed once per entry; two entries per
//           v_min3).  The lane's entries sit at fixed LDS offsets from a per-lane base
//           (without it the address arithmetic cost 2 VALU and ~60 VGPRs per entry stream).  A min over the slices gives E(v) per local scale; a DPP add with
//           the partner vector gives the group sums, whose first least entry is the ls.
//   Pass 2: the lanes re-evaluate their 64 stored dots at that ls only, and a min over the
//           slices of (error, entry) gives the lowest entry of least error.
// All arithmetic is the binary32 sequence of bq.h (explicit fma where it says fma; the file
// is compiled without contraction), so every choice matches the CPU reference bit for bit.
// With finite xn every error is finite, and min_e max(r_e, 0) = max(min_e r_e, 0), so pass 1
// clamps once at the end.  An xn that overflows makes r_e NaN exactly for the entries whose
// dot overflows (their clamped error is 0) and +inf for the rest; that rare case is handled
// by its own branch.
//
// Decoder: one lane per 8-element vector; the binary32 value d * (2 ls + 1) / 8 * q is exact.
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "bq_launch.h"

namespace bq {
namespace {

constexpr int kEntries = 512;
constexpr int kBlockElems = 256;
constexpr int kBlockBytes = 74;
constexpr int kDecodeThreads = 256;

// Grid slices per vector: 8 lanes share one vector, so a workgroup of 256 lanes holds a
// superblock's 32 vectors and each lane keeps 64 corrected dots (117 VGPRs, 4 waves per SIMD).
// 16 slices (512 lanes, 124 VGPRs, also 4 waves per SIMD) measured 18% slower at 4096 x 14336:
// the per-lane reductions and set-up double while the search work per lane halves.
constexpr int kSlices = 8;
constexpr int kThreads = (kBlockElems / 8) * kSlices;
constexpr int kPerSlice = kEntries / kSlices;
static_assert(kSlices == 8 || kSlices == 16, "slices are the lanes of a half-row or of a row");
static_assert(kEntries % kThreads == 0, "each lane stages whole grid entries");

constexpr float kMaxFinite = 0x1.fffffep127f;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], half-row mirror (lane i <-> 7 - i of
// each 8), row mirror (lane i <-> 15 - i of each 16), row rotate by 8.
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140, kRor8 = 0x128;

// Min over the kSlices lanes of a vector.
__device__ __forceinline__ float min_slices(float v) {
  v = fminf(v, dpp_f<kXor1>(v));
  v = fminf(v, dpp_f<kXor2>(v));
  v = fminf(v, dpp_f<kHalfMirror>(v));
  if constexpr (kSlices == 16) v = fminf(v, dpp_f<kMirror>(v));
  return v;
}

__device__ __forceinline__ int or_slices(int v) {
  v |= dpp_i<kXor1>(v);
  v |= dpp_i<kXor2>(v);
  v |= dpp_i<kHalfMirror>(v);
  if constexpr (kSlices == 16) v |= dpp_i<kMirror>(v);
  return v;
}

// The value of the other vector of the group (the lanes kSlices away).
__device__ __forceinline__ float partner(float v) {
  if constexpr (kSlices == 8) {
    return dpp_f<kRor8>(v);
  } else {
    // ds_swizzle bit mode inside 32 lanes: and 0x1F, or 0, xor 0x10
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  }
}

// Lexicographic min of (error, entry) over the kSlices lanes of a vector.
template <int CTRL>
__device__ __forceinline__ void key_step(float& be, int& bi) {
  const float oe = dpp_f<CTRL>(be);
  const int oi = dpp_i<CTRL>(bi);
  if (oe < be || (oe == be && oi < bi)) {
    be = oe;
    bi = oi;
  }
}

// The 8 elements of vector `vec` (elements 8 vec .. 8 vec + 7), widened exactly.
template <int DT>
__device__ __forceinline__ void load_vector(const uint8_t* __restrict__ in, int64_t vec, float* x) {
  if constexpr (DT == F32) {
    const uint4* p = reinterpret_cast<const uint4*>(in + vec * 32);
    const uint4 a = p[0], b = p[1];
    x[0] = bits_f32(a.x); x[1] = bits_f32(a.y); x[2] = bits_f32(a.z); x[3] = bits_f32(a.w);
    x[4] = bits_f32(b.x); x[5] = bits_f32(b.y); x[6] = bits_f32(b.z); x[7] = bits_f32(b.w);
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(in + vec * 16);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == BF16) {
        x[2 * i] = bits_f32(w[i] << 16);
        x[2 * i + 1] = bits_f32(w[i] & 0xffff0000u);
      } else {
        x[2 * i] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w[i] & 0xffffu));
        x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w[i] >> 16));
      }
    }
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void iq2xs_encode_kernel(const uint8_t* __restrict__ in,
                                                                const uint8_t* __restrict__ grid,
                                                                const uint16_t* __restrict__ scales,
                                                                uint8_t* __restrict__ out,
                                                                uint32_t* __restrict__ rejected) {
  __shared__ float4 s_q[2 * kEntries];  // entry e: magnitudes 0-3 at 2e, 4-7 at 2e + 1
  __shared__ float s_qn[kEntries];      // sum of squared magnitudes (exact integers)
  __shared__ uint32_t s_ls[16];
  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;
  uint8_t* dst = out + blk * kBlockBytes;
  const uint16_t dbits = scales[blk];
  const bool zero = (dbits & 0x7fffu) == 0;
  const bool bad = !zero && ((dbits & 0x7c00u) == 0x7c00u || (dbits & 0x8000u) != 0);
  if (zero || bad) {  // uniform: the all-zero superblock
    if (tid < kBlockBytes / 2) reinterpret_cast<uint16_t*>(dst)[tid] = 0;
    if (bad && tid == 0) atomicAdd(rejected, 1u);
    return;
  }

  // Stage the grid: lane t converts entries t * kStage .. t * kStage + kStage - 1.
  constexpr int kStage = kEntries / kThreads;
  {
    uint32_t w[2 * kStage];
    if constexpr (kStage == 2) {
      const uint4 g = reinterpret_cast<const uint4*>(grid)[tid];
      w[0] = g.x; w[1] = g.y; w[2] = g.z; w[3] = g.w;
    } else {
      const uint2 g = reinterpret_cast<const uint2*>(grid)[tid];
      w[0] = g.x; w[1] = g.y;
    }
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
      float q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = (float)((w[2 * k + j / 4] >> (8 * (j % 4))) & 0xffu);
      float qn = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) qn += q[j] * q[j];
      const int e = kStage * tid + k;
      s_q[2 * e] = make_float4(q[0], q[1], q[2], q[3]);
      s_q[2 * e + 1] = make_float4(q[4], q[5], q[6], q[7]);
      s_qn[e] = qn;
    }
  }

  const int lane = tid & 63;
  const int v = (tid >> 6) * (64 / kSlices) + lane / kSlices;
  const int slice = lane % kSlices;
  float a[8];
  uint32_t neg = 0;
  {
    float x[8];
    load_vector<DT>(in, blk * (kBlockElems / 8) + v, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float t = fabsf(x[j]) <= kMaxFinite ? x[j] : 0.0f;  // non-finite reads as +0
      neg |= (t < 0.0f ? 1u : 0u) << j;
      a[j] = fabsf(t);
    }
  }
  const bool odd = (__builtin_popcount(neg) & 1) != 0;
  float xn = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) xn = __builtin_fmaf(a[j], a[j], xn);

  // Per local scale l: s = d (2l + 1) / 8 (exact) and its square, wave-uniform.
  const float d = (float)__builtin_bit_cast(_Float16, dbits);
  float s2[16], sl[16];
#pragma unroll
  for (int l = 0; l < 16; ++l) {
    const float s = d * (float)(2 * l + 1) * 0.125f;
    s2[l] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, s * s)));
    sl[l] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, s)));
  }
  __syncthreads();

  // The lane's entries are slice + kSlices * i: fixed LDS offsets from a per-lane base.
  const float4* qb = s_q + 2 * slice;
  const float* qnb = s_qn + slice;

  // Pass 1.
  float E[16];
#pragma unroll
  for (int l = 0; l < 16; ++l) E[l] = __builtin_inff();
  float dots[kPerSlice];
#pragma unroll
  for (int i = 0; i < kPerSlice; i += 2) {
    float dd[2], qq[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float4 lo = qb[2 * kSlices * (i + k)], hi = qb[2 * kSlices * (i + k) + 1];
      const float q[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      float dot = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) dot = __builtin_fmaf(a[j], q[j], dot);
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = a[j] * q[j];
      const float w = fminf(fminf(fminf(p[0], p[1]), fminf(p[2], p[3])), fminf(fminf(p[4], p[5]), fminf(p[6], p[7])));
      const float fixed = __builtin_fmaf(-2.0f, w, dot);
      dots[i + k] = odd ? fixed : dot;
      dd[k] = -2.0f * dots[i + k];  // exact: fma(s, -2 dot, xn) = fma(-2s, dot, xn)
      qq[k] = qnb[kSlices * (i + k)];
    }
#pragma unroll
    for (int l = 0; l < 16; ++l) {
      const float r0 = __builtin_fmaf(s2[l], qq[0], __builtin_fmaf(sl[l], dd[0], xn));
      const float r1 = __builtin_fmaf(s2[l], qq[1], __builtin_fmaf(sl[l], dd[1], xn));
      E[l] = fminf(fminf(E[l], r0), r1);
    }
  }
#pragma unroll
  for (int l = 0; l < 16; ++l) E[l] = min_slices(E[l]);
  if (!(xn <= kMaxFinite)) {  // the same in all lanes of a vector
    int nonfinite = 0;
#pragma unroll
    for (int i = 0; i < kPerSlice; ++i) nonfinite |= (dots[i] <= kMaxFinite) ? 0 : 1;
    nonfinite = or_slices(nonfinite);
#pragma unroll
    for (int l = 0; l < 16; ++l) E[l] = nonfinite ? 0.0f : __builtin_inff();
  }
  int bl = 0;
  float bg = 0.0f;
#pragma unroll
  for (int l = 0; l < 16; ++l) {
    const float e = fmaxf(E[l], 0.0f);
    const float g = e + partner(e);  // fl(E(v0) + E(v1)), the same in both vectors' lanes
    if (l == 0 || g < bg) {
      bg = g;
      bl = l;
    }
  }

  // Pass 2.
  const float s = d * (float)(2 * bl + 1) * 0.125f;
  const float ss = s * s, m2 = -2.0f * s;
  float be = 0.0f;
  int bi = 0;
#pragma unroll
  for (int i = 0; i < kPerSlice; ++i) {
    const float r = fmaxf(__builtin_fmaf(ss, qnb[kSlices * i], __builtin_fmaf(m2, dots[i], xn)), 0.0f);
    if (i == 0 || r < be) {
      be = r;
      bi = i;
    }
  }
  bi = slice + kSlices * bi;
  key_step<kXor1>(be, bi);
  key_step<kXor2>(be, bi);
  key_step<kHalfMirror>(be, bi);
  if constexpr (kSlices == 16) key_step<kMirror>(be, bi);

  if (slice == 0) {
    uint32_t mask = neg;
    if (odd) {  // flip the first element of least |x_j| q_j
      const float4 lo = s_q[2 * bi], hi = s_q[2 * bi + 1];
      const float q[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = a[j] * q[j];
      const float w = fminf(fminf(fminf(p[0], p[1]), fminf(p[2], p[3])), fminf(fminf(p[4], p[5]), fminf(p[6], p[7])));
      int k = 7;
#pragma unroll
      for (int j = 6; j >= 0; --j) k = p[j] == w ? j : k;
      mask ^= 1u << k;
    }
    *reinterpret_cast<uint16_t*>(dst + 2 + 2 * v) = (uint16_t)(bi | ((mask & 0x7fu) << 9));
    if ((v & 1) == 0) s_ls[v >> 1] = (uint32_t)bl;
  }
  __syncthreads();
  if (tid < 8) dst[66 + tid] = (uint8_t)(s_ls[2 * tid] | (s_ls[2 * tid + 1] << 4));
  if (tid == 8) *reinterpret_cast<uint16_t*>(dst) = dbits;
}

// The 8 values of vector `vec` in the output type, stored non-temporally (consecutive lanes
// write consecutive 16 bytes; at 4096 x 14336 to bf16 the decoders took 6-8% less time than
// with ordinary stores).
template <int DT>
__device__ __forceinline__ void store_vector(uint8_t* out, int64_t vec, float* v) {
  if constexpr (DT == F32) {
    typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
    u32x4_nt* p = reinterpret_cast<u32x4_nt*>(out + vec * 32);
    const u32x4_nt q0 = {f32_bits(v[0]), f32_bits(v[1]), f32_bits(v[2]), f32_bits(v[3])};
    const u32x4_nt q1 = {f32_bits(v[4]), f32_bits(v[5]), f32_bits(v[6]), f32_bits(v[7])};
    __builtin_nontemporal_store(q0, p);
    __builtin_nontemporal_store(q1, p + 1);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // Values are held in registers before the conversion: folded into it, a negated product
      // becomes a mixed-precision fma with a +0 addend, which would turn -0 into +0.
      float x0 = v[2 * i], x1 = v[2 * i + 1];
      asm("" : "+v"(x0), "+v"(x1));
      uint16_t lo, hi;
      if constexpr (DT == BF16) {
        lo = __builtin_bit_cast(uint16_t, (__bf16)x0);
        hi = __builtin_bit_cast(uint16_t, (__bf16)x1);
      } else {
        lo = __builtin_bit_cast(uint16_t, (_Float16)x0);
        hi = __builtin_bit_cast(uint16_t, (_Float16)x1);
      }
      w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
    const u32x4_nt q = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(q, reinterpret_cast<u32x4_nt*>(out + vec * 16));
  }
}

template <int DT>
__global__ __launch_bounds__(kDecodeThreads) void iq2xs_decode_kernel(const uint8_t* __restrict__ blocks,
                                                                const uint8_t* __restrict__ grid, int64_t nvec,
                                                                uint8_t* __restrict__ out) {
  const int64_t vec = (int64_t)blockIdx.x * kDecodeThreads + threadIdx.x;
  if (vec >= nvec) return;
  const uint8_t* blk = blocks + (vec >> 5) * kBlockBytes;
  const int v = (int)(vec & 31);
  const uint16_t dbits = *reinterpret_cast<const uint16_t*>(blk);
  const uint32_t word = *reinterpret_cast<const uint16_t*>(blk + 2 + 2 * v);
  const int g = v >> 1;
  const int ls = (blk[66 + (g >> 1)] >> (4 * (g & 1))) & 15;
  const float dl = (float)__builtin_bit_cast(_Float16, dbits) * (float)(2 * ls + 1) * 0.125f;
  const uint32_t s7 = word >> 9;
  const uint32_t signs = s7 | ((uint32_t)(__builtin_popcount(s7) & 1) << 7);
  const uint2 q = *reinterpret_cast<const uint2*>(grid + 8 * (word & 511u));
  float val[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float t = dl * (float)(((j < 4 ? q.x : q.y) >> (8 * (j & 3))) & 0xffu);
    val[j] = ((signs >> j) & 1u) ? -t : t;
  }
  store_vector<DT>(out, vec, val);
}

template <int DT>
hipError_t launch_encode_dt(const void* in, int64_t n, const uint8_t* grid, const uint16_t* scales, uint8_t* blocks,
                            uint32_t* rejected, hipStream_t s) {
  return launch_kernel(iq2xs_encode_kernel<DT>, dim3((unsigned)(n / kBlockElems)), dim3(kThreads), s,
                       static_cast<const uint8_t*>(in), grid, scales, blocks, rejected);
}

template <int DT>
hipError_t launch_decode_dt(const uint8_t* blocks, const uint8_t* grid, int64_t n, void* out, hipStream_t s) {
  const int64_t nvec = n / 8;
  return launch_kernel(iq2xs_decode_kernel<DT>, dim3((unsigned)((nvec + kDecodeThreads - 1) / kDecodeThreads)),
                       dim3(kDecodeThreads),
                       s, blocks, grid, nvec, static_cast<uint8_t*>(out));
}

}  // namespace

int launch_iq2xs_quantize(const void* in, int dtype, int64_t n, const uint8_t* grid, const uint16_t* scales,
                          uint8_t* blocks, uint32_t* rejected, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == F32) return (int)launch_encode_dt<F32>(in, n, grid, scales, blocks, rejected, s);
  if (dtype == F16) return (int)launch_encode_dt<F16>(in, n, grid, scales, blocks, rejected, s);
  return (int)launch_encode_dt<BF16>(in, n, grid, scales, blocks, rejected, s);
}

int launch_iq2xs_dequantize(const uint8_t* blocks, const uint8_t* grid, int64_t n, int dtype, void* out,
                            void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == F32) return (int)launch_decode_dt<F32>(blocks, grid, n, out, s);
  if (dtype == F16) return (int)launch_decode_dt<F16>(blocks, grid, n, out, s);
  return (int)launch_decode_dt<BF16>(blocks, grid, n, out, s);
}

}  // namespace bq
