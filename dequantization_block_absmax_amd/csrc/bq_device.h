// bq_device.h -- device helpers shared by the quantize and statistics kernels: the
// per-workgroup LUT of the nearest-code search and the search itself.  The bucket functions
// and the LUT contents are described in bq_internal.h.
#pragma once

#include <hip/hip_runtime.h>

#include "bq_internal.h"

namespace bq {

template <int M>
struct Entry { typedef uint4 type; };
template <>
struct Entry<1> { typedef uint2 type; };

// LDS size of the LUT, in entries.
template <int MODE, int M>
struct LutLayout {
  static constexpr int kSize = MODE == LIN ? kLinLutMax : MODE == LOG ? kLutMax : MODE == F16B ? kF16Size : 1;
};

// Nearest code of y (see bq_internal.h for the bucket functions).  y must be in [-1, 1] for
// LIN; LOG and SEARCH also take a non-finite y, which gives z.
template <int MODE, int M>
__device__ __forceinline__ uint32_t nearest_code(float y, const QuantArgs& qa,
                                                 const typename Entry<M>::type* lut,
                                                 const float* s_thr) {
  if constexpr (MODE == SEARCH) {
    if (!(fabsf(y) <= 1.0f)) return (uint32_t)qa.z;
    int q = 0;
    for (int step = qa.K >> 1; step >= 1; step >>= 1) q += (y >= s_thr[q + step - 1]) ? step : 0;
    return (uint32_t)q;
  } else {
    typename Entry<M>::type e;
    if constexpr (MODE == LIN) {
      // zz is the integer 2^23 + bucket, so its bits give the entry's byte offset in one
      // shift-and-add (lin_off removes the bits of 2^23).
      constexpr int kLog2E = M == 1 ? 3 : 4;
      const float zz = __builtin_fmaf(y, qa.lin_scale, qa.lin_bias);
      const uint32_t off = (f32_bits(zz) << kLog2E) + qa.lin_off;
      e = *reinterpret_cast<const typename Entry<M>::type*>(reinterpret_cast<const char*>(lut) + off);
    } else if constexpr (MODE == F16B) {
      static_assert(M == 1, "F16B entries are 8 bytes");
      typedef __fp16 h2 __attribute__((ext_vector_type(2)));
      const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(y, 0.0f));
      const uint32_t m = (d & 0x3ff0u) | ((d >> 1) & 0x4000u);
      e = *reinterpret_cast<const typename Entry<M>::type*>(reinterpret_cast<const char*>(lut) + (m >> 1));
    } else {
      // Byte offset of the entry, in five operations: LO and HI are multiples of 2^SH, so
      // clamping |y| bits >> SH to [LO >> SH, HI >> SH] gives j + (LO >> SH); the sign picks the
      // bias that removes LO >> SH and, for negative y, adds the NJ buckets of the positive side.
      constexpr int kLog2E = M == 1 ? 3 : 4;
      const uint32_t u = f32_bits(y);
      uint32_t j = __builtin_amdgcn_ubfe(u, (uint32_t)qa.sh, (uint32_t)(31 - qa.sh));
      asm("v_med3_u32 %0, %1, %2, %3" : "=v"(j) : "v"(j), "v"(qa.jlo), "v"(qa.jhi));
      const uint32_t neg = (uint32_t)((int32_t)u >> 31);
      const uint32_t bias = (neg & qa.log_nbias) | (~neg & qa.log_bias);
      const uint32_t off = (j << kLog2E) + bias;
      e = *reinterpret_cast<const typename Entry<M>::type*>(reinterpret_cast<const char*>(lut) + off);
    }
    uint32_t q = e.x + (y >= bits_f32(e.y) ? 1u : 0u);
    if constexpr (M >= 2) q += (y >= bits_f32(e.z) ? 1u : 0u);
    if constexpr (M >= 3) q += (y >= bits_f32(e.w) ? 1u : 0u);
    return q;
  }
}

// Code from a fetched LUT entry (base, then up to three thresholds).
template <int M>
__device__ __forceinline__ uint32_t entry_code(float y, const typename Entry<M>::type& e) {
  uint32_t q = e.x + (y >= bits_f32(e.y) ? 1u : 0u);
  if constexpr (M >= 2) q += (y >= bits_f32(e.z) ? 1u : 0u);
  if constexpr (M >= 3) q += (y >= bits_f32(e.w) ? 1u : 0u);
  return q;
}

// Nearest codes of two values y0, y1 in [-1, 1].  F16B converts both in one instruction and
// works on the pair h0 | h1 << 16: a mask keeps bits 4..13 of each half, the sign bits
// shifted right by one land in the cleared bits 14 and 30 (one and-or), and the
// 8-byte entries' offsets are (h0' >> 4) * 8 = bits 1..15 and (h1' >> 4) * 8 = the word >> 17.
// Other modes take the values one at a time.
template <int MODE, int M>
__device__ __forceinline__ void nearest_pair(float y0, float y1, const QuantArgs& qa,
                                             const typename Entry<M>::type* lut, const float* s_thr,
                                             uint32_t& q0, uint32_t& q1) {
  if constexpr (MODE == F16B) {
    static_assert(M == 1, "F16B entries are 8 bytes");
    typedef __fp16 h2 __attribute__((ext_vector_type(2)));
    const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(y0, y1));
    uint32_t m = d & 0x3ff03ff0u;
    uint32_t t = d >> 1;
    asm("" : "+v"(m), "+v"(t));  // one mask and one shift for both halves (the compiler would
                                 // otherwise split them per half)
    const uint32_t p = (t & 0x40004000u) | m;  // bits 14 and 30 of m are clear: one v_and_or
    const uint32_t off0 = __builtin_amdgcn_ubfe(p, 1u, 15u);
    const uint32_t off1 = p >> 17;
    const char* base = reinterpret_cast<const char*>(lut);
    const typename Entry<M>::type e0 = *reinterpret_cast<const typename Entry<M>::type*>(base + off0);
    const typename Entry<M>::type e1 = *reinterpret_cast<const typename Entry<M>::type*>(base + off1);
    q0 = entry_code<M>(y0, e0);
    q1 = entry_code<M>(y1, e1);
  } else {
    q0 = nearest_code<MODE, M>(y0, qa, lut, s_thr);
    q1 = nearest_code<MODE, M>(y1, qa, lut, s_thr);
  }
}

// Maximum of v over aligned groups of g lanes (g a power of two, 1..64, the same in every
// lane), returned in every lane of the group.  Inside a 16-lane row the exchanges are DPP
// lane permutes (xor 1 and xor 2 by quad permutes, then the half-row and row mirrors, which
// pair each 4- and 8-lane group with its neighbour); wider groups add one cross-row shuffle
// and two lane reads.  Each DPP step is one instruction with a short latency, where an LDS
// shuffle costs an address computation and a round trip through the LDS unit.
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v, int g) {
  if (g >= 2) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
  if (g >= 4) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
  if (g >= 8) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
  if (g >= 16) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
  if (g >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  if (g >= 64) v = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
  return v;
}

// Maximum of v over the whole wave, returned in every lane: the DPP steps of group_max_u32
// leave each 16-lane row's maximum in all its lanes, and four lane reads join the rows.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// One output word from its codes, in byte order: eight 4-bit codes (the first element of a
// pair in the high nibble) or four 8-bit codes.  The bytes are joined with byte permutes, one
// operation per byte pair, where a chain of shifts and ORs is compiled into more operations.
template <int KB>
__device__ __forceinline__ uint32_t pack_word(const uint32_t* q) {
  uint32_t b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) b[k] = KB == 4 ? (q[2 * k] << 4) | q[2 * k + 1] : q[k];
  const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);  // b0 | b1 << 8
  const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);  // b2 | b3 << 8
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);                    // lo | hi << 16
}

// The table words one thread copies into LDS: thresholds and per-bucket bases, read from the
// kernel arguments in one batch with fixed trip counts, so the prologue waits for memory once.
// A kernel issues these loads before its first data loads: loads return in issue order, so the
// LUT fill need not wait behind the data.
template <int MODE, int M, int NT>
struct LutWords {
  static constexpr int kThrIt = (260 + NT - 1) / NT;
  static constexpr int kLutIt = MODE == SEARCH ? 0 : (LutLayout<MODE, M>::kSize + NT - 1) / NT;
  float th[kThrIt];
  uint32_t bs[kLutIt > 0 ? kLutIt : 1];
};

template <int MODE, int M, int NT>
__device__ __forceinline__ LutWords<MODE, M, NT> lut_fetch(const QuantArgs& qa, int tid) {
  using L = LutWords<MODE, M, NT>;
  L l;
#pragma unroll
  for (int k = 0; k < L::kThrIt; ++k) {
    const int i = tid + k * NT;
    l.th[k] = i < 260 ? qa.thr[i] : 0.0f;
  }
  // Every entry of the base array is read, not just the nbuckets in use: the host zero-fills
  // the rest, and a bound known at compile time leaves no branch between the loads.  F16B
  // entries of negative y (index 1024 on) take their base from index - 63, and the hole reads
  // a valid index.
  constexpr int kSize = LutLayout<MODE, M>::kSize;
#pragma unroll
  for (int k = 0; k < L::kLutIt; ++k) {
    const int i = tid + k * NT;
    if constexpr (MODE == F16B) {
      const int j = i >= kF16NegLo ? i - kF16NegBase : min(i, kF16Pos - 1);
      l.bs[k] = (k + 1) * NT <= kSize || i < kSize ? qa.base[j] : 0u;
    } else {
      l.bs[k] = (k + 1) * NT <= kSize || i < kSize ? qa.base[i] : 0u;
    }
  }
  return l;
}

// Writes the thresholds into LDS and expands the per-bucket bases into LDS entries
// (base, T[base], T[base+1], T[base+2]); special buckets get (z, NaN, ...).
// s_lut holds LutLayout<MODE, M>::kSize entries.
// Must be called by every thread of the workgroup; ends with a barrier.
template <int MODE, int M, int NT>
__device__ __forceinline__ void lut_fill(const QuantArgs& qa, const LutWords<MODE, M, NT>& l,
                                         typename Entry<M>::type* s_lut, float* s_thr, int tid) {
  using E = typename Entry<M>::type;
  using L = LutWords<MODE, M, NT>;
#pragma unroll
  for (int k = 0; k < L::kThrIt; ++k)
    if (tid + k * NT < 260) s_thr[tid + k * NT] = l.th[k];
  __syncthreads();
  if constexpr (MODE != SEARCH) {
    // Rounds of NT entries: a round that starts past nbuckets is skipped (a uniform test);
    // inside a round every entry is written (those past nbuckets from the zero bases are never
    // read), so the threshold reads and entry writes form one batch instead of a chain of
    // branches.
    constexpr int kSize = LutLayout<MODE, M>::kSize;
#pragma unroll
    for (int k = 0; k < L::kLutIt; ++k) {
      const int i = tid + k * NT;
      // F16B: rounds wholly inside the hole (never read) are skipped too
      const bool hole = MODE == F16B && k * NT >= kF16Pos && (k + 1) * NT <= kF16NegLo;
      if (!hole && k * NT < qa.nbuckets && ((k + 1) * NT <= kSize || i < kSize)) {
        const uint32_t b = l.bs[k];  // <= 255, so b + 2 stays inside the 260 thresholds
        E e;
        e.x = b;
        e.y = f32_bits(s_thr[b]);
        if constexpr (M >= 2) {
          e.z = f32_bits(s_thr[b + 1]);
          e.w = f32_bits(s_thr[b + 2]);
        }
        s_lut[i] = e;
      }
    }
    // The two special buckets are rewritten by the threads that wrote them above, so program
    // order puts these writes last: code z, and NaN thresholds that no compare passes.
    E sp;
    sp.x = (uint32_t)qa.z;
    sp.y = 0x7fc00000u;
    if constexpr (M >= 2) sp.z = sp.w = 0x7fc00000u;
    if (qa.special0 >= 0 && tid == (qa.special0 & (NT - 1))) s_lut[qa.special0] = sp;
    if (qa.special1 >= 0 && tid == (qa.special1 & (NT - 1))) s_lut[qa.special1] = sp;
    __syncthreads();
  }
}

}  // namespace bq
