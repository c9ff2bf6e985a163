// k_iq1s.hip -- IQ1_S-style encoding and decoding of 256-element superblocks
// ("[OMNIML-5899] Add CUDA kernels for IQ packing", Model-Optimizer PR 2448: "Provenance"
// (16.875 = 15 x (1 + 1/8), the 0.61 predictor, the 0.125 delta), the review items "Wire
// format", "Scale anchors" and "Search equivalence", and the round-3 item on the shifted
// objective).  The byte layout and the search are stated in bq.h.
//
// Encoder: one 256-lane workgroup per superblock; lane (wave w, lane l) serves vector
// v = 8w + l / 8 and grid slice k = l % 8 (entries k, k + 8, ..., k + 2040).  The grid sits in
// LDS as binary16 (exact for signed bytes: the fma takes it without a conversion) with the two
// shifted norms of each entry (qn + 2 delta qs + 8 delta^2 for delta = +-1/8, exact).
//   Scale: the superblock maximum of |x| (DPP within waves, LDS across), then the binary32
//          quotient and product and the binary16 rounding, saturated.
//   Pass 1: per entry the fma-chain dot, the two shifted dots fma(+-1/8, xsum, dot), and for
//           each of the 16 choices (ls, sign) the error's two fmas (with -2 * sdot formed
//           once: fma(dl, -2 sdot, xn) equals fma(-2 dl, sdot, xn) bit for bit), two entries
//           per v_min3.  A min over the slices gives each vector's 16 errors; the four
//           vectors of a sub-block are summed in vector order through LDS, and every lane of
//           the sub-block takes the first least choice.
//   Pass 2: the lanes recompute their entries' dots at that choice only (storing 256 per
//           lane does not fit), and a min over the slices of (error, entry) gives the lowest
//           entry of least error.
// As in the IQ2_XS encoder, finite xn keeps every error finite, so pass 1 clamps once at the
// end; an xn that overflows makes an error NaN exactly where the shifted dot is +inf or NaN
// (its clamped error is 0) and +inf elsewhere, which a rare branch reproduces per sign.
//
// Decoder: one lane per 8-element vector (four vectors per lane, 256 apart): d * (2 ls + 1)
// (exact) times (g + delta) (exact), rounded once to binary32 and once to the output type.
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "bq_launch.h"

namespace bq {
namespace {

constexpr int kEntries = 2048;
constexpr int kBlockElems = 256;
constexpr int kBlockBytes = 50;
constexpr int kThreads = 256;
constexpr int kSlices = 8;
constexpr int kPerSlice = kEntries / kSlices;
constexpr int kDecodeThreads = 256;
// Vectors per decoder lane, 256 apart (8.2% faster than one at 4096 x 14336 to bf16; eight
// were slower)
constexpr int kDecVPL = 4;
static_assert(kThreads == (kBlockElems / 8) * kSlices, "one lane per (vector, slice)");
static_assert(kEntries % kThreads == 0, "each lane stages whole grid entries");

constexpr float kMaxFinite = 0x1.fffffep127f;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

__device__ __forceinline__ float min8(float v) {
  v = fminf(v, dpp_f<kXor1>(v));
  v = fminf(v, dpp_f<kXor2>(v));
  return fminf(v, dpp_f<kHalfMirror>(v));
}
__device__ __forceinline__ int or8(int v) {
  v |= dpp_i<kXor1>(v);
  v |= dpp_i<kXor2>(v);
  return v | dpp_i<kHalfMirror>(v);
}
template <int CTRL>
__device__ __forceinline__ void key_step(float& be, int& bi) {
  const float oe = dpp_f<CTRL>(be);
  const int oi = dpp_i<CTRL>(bi);
  if (oe < be || (oe == be && oi < bi)) {
    be = oe;
    bi = oi;
  }
}

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

// Dot of the lane's vector with one entry: fma chain from +0, j ascending.
__device__ __forceinline__ float entry_dot(const float* x, const h8 q) {
  float dot = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) dot = __builtin_fmaf(x[j], (float)q[j], dot);
  return dot;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void iq1s_encode_kernel(const uint8_t* __restrict__ in,
                                                               const int8_t* __restrict__ grid,
                                                               uint8_t* __restrict__ out) {
  __shared__ h8 s_q[kEntries];         // entry e: its 8 signed bytes as binary16
  __shared__ float2 s_sn[kEntries];    // shifted norms for delta = +1/8 and -1/8
  __shared__ float s_E[32 * 16];       // per vector, its least error for each choice
  __shared__ float s_max[kThreads / 64];
  __shared__ uint32_t s_hi[32];
  __shared__ uint32_t s_choice[8];
  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x;
  uint8_t* dst = out + blk * kBlockBytes;

  // Stage the grid: lane t converts entries 8t .. 8t + 7.
  constexpr int kStage = kEntries / kThreads;
#pragma unroll
  for (int k = 0; k < kStage; k += 2) {
    const uint4 g = reinterpret_cast<const uint4*>(grid)[tid * (kStage / 2) + k / 2];
    const uint32_t w[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      h8 q;
      float qn = 0.0f, qs = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int v = (int)(int8_t)(w[2 * h + j / 4] >> (8 * (j % 4)));
        q[j] = (_Float16)v;
        qn += (float)(v * v);
        qs += (float)v;
      }
      const int e = tid * kStage + k + h;
      s_q[e] = q;
      // qn + 2 delta qs + 8 delta^2, exact (qn, qs integers of at most 17 bits)
      s_sn[e] = make_float2(qn + 0.25f * qs + 0.125f, qn - 0.25f * qs + 0.125f);
    }
  }

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int v = wave * 8 + (lane >> 3);
  const int slice = lane & 7;
  float x[8];
  {
    float raw[8];
    load_vector<DT>(in, blk * (kBlockElems / 8) + v, raw);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = fabsf(raw[j]) <= kMaxFinite ? raw[j] : 0.0f;  // non-finite reads as +0
  }
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[j]));
  am = fmaxf(am, dpp_f<kXor1>(am));
  am = fmaxf(am, dpp_f<kXor2>(am));
  am = fmaxf(am, dpp_f<kHalfMirror>(am));
  am = fmaxf(am, dpp_f<kMirror>(am));
  am = fmaxf(am, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, am), 0x401F)));
  am = fmaxf(am, __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, am), 32)));
  if (lane == 0) s_max[wave] = am;
  __syncthreads();  // also completes the grid staging
  float amax = s_max[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) amax = fmaxf(amax, s_max[w]);
  const float dq = (amax / 16.875f) * 0.61f;
  uint16_t dbits = __builtin_bit_cast(uint16_t, (_Float16)dq);
  if ((dbits & 0x7c00u) == 0x7c00u) dbits = 0x7bff;  // saturate (amax is finite)
  if ((dbits & 0x7fffu) == 0) {                     // uniform: the all-zero superblock
    if (tid < kBlockBytes / 2) reinterpret_cast<uint16_t*>(dst)[tid] = 0;
    return;
  }
  const float d = (float)__builtin_bit_cast(_Float16, dbits);

  float xn = 0.0f, xsum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    xn = __builtin_fmaf(x[j], x[j], xn);
    xsum = __builtin_fmaf(x[j], 1.0f, xsum);
  }
  // dl = d (2 ls + 1) (exact) and dl * dl, wave-uniform.
  float dl[8], dl2[8];
#pragma unroll
  for (int l = 0; l < 8; ++l) {
    const float t = d * (float)(2 * l + 1);
    dl[l] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, t)));
    dl2[l] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, t * t)));
  }

  const h8* qb = s_q + slice;
  const float2* snb = s_sn + slice;

  // Pass 1: E[c], c = ls + 8 * sign (sign 1: delta = -1/8).
  float E[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) E[c] = __builtin_inff();
#pragma unroll 2
  for (int i = 0; i < kPerSlice; i += 2) {
    float np[2], nm[2], sp[2], sm[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float dot = entry_dot(x, qb[kSlices * (i + k)]);
      const float2 sn = snb[kSlices * (i + k)];
      np[k] = -2.0f * __builtin_fmaf(0.125f, xsum, dot);   // -2 sdot, exact doubling
      nm[k] = -2.0f * __builtin_fmaf(-0.125f, xsum, dot);
      sp[k] = sn.x;
      sm[k] = sn.y;
    }
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      const float p0 = __builtin_fmaf(dl2[l], sp[0], __builtin_fmaf(dl[l], np[0], xn));
      const float p1 = __builtin_fmaf(dl2[l], sp[1], __builtin_fmaf(dl[l], np[1], xn));
      E[l] = fminf(fminf(E[l], p0), p1);
      const float m0 = __builtin_fmaf(dl2[l], sm[0], __builtin_fmaf(dl[l], nm[0], xn));
      const float m1 = __builtin_fmaf(dl2[l], sm[1], __builtin_fmaf(dl[l], nm[1], xn));
      E[8 + l] = fminf(fminf(E[8 + l], m0), m1);
    }
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) E[c] = min8(E[c]);
  if (!(xn <= kMaxFinite)) {  // the same in the 8 lanes of a vector
    int np_nf = 0, nm_nf = 0;
    for (int i = 0; i < kPerSlice; ++i) {
      const float dot = entry_dot(x, qb[kSlices * i]);
      np_nf |= (__builtin_fmaf(0.125f, xsum, dot) <= kMaxFinite) ? 0 : 1;
      nm_nf |= (__builtin_fmaf(-0.125f, xsum, dot) <= kMaxFinite) ? 0 : 1;
    }
    np_nf = or8(np_nf);
    nm_nf = or8(nm_nf);
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      E[l] = np_nf ? 0.0f : __builtin_inff();
      E[8 + l] = nm_nf ? 0.0f : __builtin_inff();
    }
  }
  if (slice == 0) {
#pragma unroll
    for (int c = 0; c < 16; ++c) s_E[v * 16 + c] = fmaxf(E[c], 0.0f);
  }
  __syncthreads();
  const int sb = v >> 2;  // 32-element sub-block
  int bc = 0;
  float bsum = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    float sum = s_E[(4 * sb) * 16 + c];
#pragma unroll
    for (int l = 1; l < 4; ++l) sum += s_E[(4 * sb + l) * 16 + c];  // vector order
    if (c == 0 || sum < bsum) {
      bsum = sum;
      bc = c;
    }
  }

  // Pass 2.
  const float dls = d * (float)(2 * (bc & 7) + 1);
  const float dls2 = dls * dls, m2 = -2.0f * dls;
  const float delta = (bc & 8) ? -0.125f : 0.125f;
  const float* snsel = reinterpret_cast<const float*>(snb) + ((bc & 8) ? 1 : 0);
  float be = 0.0f;
  int bi = 0;
  for (int i = 0; i < kPerSlice; ++i) {
    const float sdot = __builtin_fmaf(delta, xsum, entry_dot(x, qb[kSlices * i]));
    const float r = fmaxf(__builtin_fmaf(dls2, snsel[2 * kSlices * i], __builtin_fmaf(m2, sdot, xn)), 0.0f);
    if (i == 0 || r < be) {
      be = r;
      bi = i;
    }
  }
  bi = slice + kSlices * bi;
  key_step<kXor1>(be, bi);
  key_step<kXor2>(be, bi);
  key_step<kHalfMirror>(be, bi);

  if (slice == 0) {
    dst[2 + v] = (uint8_t)(bi & 0xff);
    s_hi[v] = (uint32_t)(bi >> 8);
    if ((v & 3) == 0) s_choice[sb] = (uint32_t)bc;
  }
  __syncthreads();
  if (tid < 8) {  // qh of sub-block tid: the four vectors' high index bits, ls, delta sign
    const uint32_t c = s_choice[tid];
    const uint32_t qh = s_hi[4 * tid] | (s_hi[4 * tid + 1] << 3) | (s_hi[4 * tid + 2] << 6) |
                        (s_hi[4 * tid + 3] << 9) | ((c & 7u) << 12) | ((c >> 3) << 15);
    *reinterpret_cast<uint16_t*>(dst + 34 + 2 * tid) = (uint16_t)qh;
  }
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
      // held in registers before the conversion, so that it is not fused with the product
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
__global__ __launch_bounds__(kDecodeThreads) void iq1s_decode_kernel(const uint8_t* __restrict__ blocks,
                                                                     const int8_t* __restrict__ grid, int64_t nvec,
                                                                     uint8_t* __restrict__ out) {
#pragma unroll
  for (int k = 0; k < kDecVPL; ++k) {
    const int64_t vec0 = ((int64_t)blockIdx.x * kDecVPL + k) * kDecodeThreads + threadIdx.x;
    const int64_t vec = min(vec0, nvec - 1);
    const uint8_t* blk = blocks + (vec >> 5) * kBlockBytes;
    const int v = (int)(vec & 31);
    const uint16_t dbits = *reinterpret_cast<const uint16_t*>(blk);
    const uint32_t qh = *reinterpret_cast<const uint16_t*>(blk + 34 + 2 * (v >> 2));
    const uint32_t e = blk[2 + v] | (((qh >> (3 * (v & 3))) & 7u) << 8);
    const float dl = (float)__builtin_bit_cast(_Float16, dbits) * (float)(2 * ((qh >> 12) & 7u) + 1);
    const float delta = (qh & 0x8000u) ? -0.125f : 0.125f;
    const uint2 g = *reinterpret_cast<const uint2*>(grid + 8 * e);
    float val[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = (int)(int8_t)((j < 4 ? g.x : g.y) >> (8 * (j & 3)));
      val[j] = dl * ((float)q + delta);
    }
    if (vec0 < nvec) store_vector<DT>(out, vec0, val);
  }
}

template <int DT>
hipError_t launch_encode_dt(const void* in, int64_t n, const int8_t* grid, uint8_t* blocks, hipStream_t s) {
  return launch_kernel(iq1s_encode_kernel<DT>, dim3((unsigned)(n / kBlockElems)), dim3(kThreads), s,
                       static_cast<const uint8_t*>(in), grid, blocks);
}

template <int DT>
hipError_t launch_decode_dt(const uint8_t* blocks, const int8_t* grid, int64_t n, void* out, hipStream_t s) {
  const int64_t nvec = n / 8;
  return launch_kernel(iq1s_decode_kernel<DT>,
                       dim3((unsigned)((nvec + kDecodeThreads * kDecVPL - 1) / (kDecodeThreads * kDecVPL))),
                       dim3(kDecodeThreads), s, blocks, grid, nvec, static_cast<uint8_t*>(out));
}

}  // namespace

int launch_iq1s_quantize(const void* in, int dtype, int64_t n, const int8_t* grid, uint8_t* blocks, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == F32) return (int)launch_encode_dt<F32>(in, n, grid, blocks, s);
  if (dtype == F16) return (int)launch_encode_dt<F16>(in, n, grid, blocks, s);
  return (int)launch_encode_dt<BF16>(in, n, grid, blocks, s);
}

int launch_iq1s_dequantize(const uint8_t* blocks, const int8_t* grid, int64_t n, int dtype, void* out,
                           void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == F32) return (int)launch_decode_dt<F32>(blocks, grid, n, out, s);
  if (dtype == F16) return (int)launch_decode_dt<F16>(blocks, grid, n, out, s);
  return (int)launch_decode_dt<BF16>(blocks, grid, n, out, s);
}

}  // namespace bq
