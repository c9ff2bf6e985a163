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
// one LDS exchange between the two waves.  A 256-lane workgroup quantizes one tile of 8192
// elements.  With 16-bit input, 8-bit codes and blocks of 2048 or more, a whole tile takes an
// interleaved chunk instead (load_chunk_il: each of the wave's four loads reads 1 KB of
// consecutive bytes and each code store writes 512), which needs no LDS exchange for the
// stores (bf16 2^26, B = 4096, with the non-temporal loads: 33.8 against 37.4 us, identical
// output).  (Workgroups that
// each took several tiles, with the next tile's loads issued ahead of the current tile's
// arithmetic, measured slower on MI355X: 41.2 against 36.9 us for 2^26 bf16 elements with
// 8-bit codes, B = 4096; the second register buffer costs more occupancy than the overlap
// gains.)
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Non-temporal 16-byte store of the codes: they stream to memory without displacing the input
// from the caches (2^29 bf16, 4-bit: 224 us against 234 us with ordinary stores on MI355X; the
// same hint on the absmax stores measured slower).  The hint suits loads only where each load
// instruction of a wave reads whole cache lines (the LDS-transposed and interleaved chunks):
// on lane-contiguous chunks, whose lines are shared by four instructions, it doubled the time.
__device__ __forceinline__ void store16_nt(uint8_t* p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

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

// Max of the finite-|x| key over the lane chunk; *finite tells whether every element of the
// chunk is finite.  Common case first: the max of 2|x| (the shift drops the sign), for 16-bit
// input two packed operations per pair.  Only when a wave holds an Inf/NaN (exponent all ones)
// is the key recomputed with the wrap that excludes non-finite elements; for finite elements
// both give 2|x| + off.
template <int DT>
__device__ __forceinline__ uint32_t chunk_key(const uint32_t* w, bool* finite) {
  if constexpr (DT == F32) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = max(m, w[i] << 1);
    *finite = m < 0xff000000u;
    // wave-uniform, so the rare path is a branch the common case skips
    if (__builtin_expect(__all(*finite), 1)) return m + 0x01000000u;
    uint32_t k = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) k = max(k, (w[i] << 1) + 0x01000000u);
    return k;
  } else {
    constexpr unsigned short off = DT == BF16 ? 0x0100 : 0x0800;
    constexpr uint32_t kNonFinite = DT == BF16 ? 0xff00u : 0xf800u;  // 2 * (bits of +Inf)
    u16x2 acc = {0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, w[i]) << (u16x2){1, 1});
    const uint32_t m = max((uint32_t)acc.x, (uint32_t)acc.y);
    *finite = m < kNonFinite;
    if (__builtin_expect(__all(*finite), 1)) return m + off;
    acc = (u16x2){0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const u16x2 h = __builtin_bit_cast(u16x2, w[i]);
      acc = __builtin_elementwise_max(acc, (h << (u16x2){1, 1}) + (u16x2){off, off});
    }
    return max((uint32_t)acc.x, (uint32_t)acc.y);
  }
}

// The block absmax in the input's own 16-bit format (fp16 / bf16 input), from the max key: the
// maximum of |x| over elements of that format is itself a value of the format, so the 16 bits
// hold it exactly.  +0 when the block has no finite element.
template <int DT>
__device__ __forceinline__ uint32_t key_to_bits16(uint32_t k) {
  constexpr uint32_t off = DT == BF16 ? 0x0100u : 0x0800u;
  return k >= off ? (k - off) >> 1 : 0u;
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

// Interleaved chunk (16-bit input, 8-bit codes, blocks of 2048 or more): the lane's 32
// elements are 8 consecutive ones from each of the wave's four 512-element segments, so that
// each of the four 16-byte loads of the wave reads 1 KB of consecutive bytes and each 8-byte
// store of codes writes 512.  The wave's 2048 elements lie in one block either way.  Loads and
// stores are non-temporal, as in the 4-bit path (bf16 2^26, B = 4096: 33.8 against 35.1 us with
// ordinary loads, and 37.4 without the interleaving).
template <int DT>
__device__ __forceinline__ void load_chunk_il(const uint8_t* __restrict__ in, int64_t wave0, int lane, uint32_t* w) {
  const uint4* src = reinterpret_cast<const uint4*>(in + (wave0 + 8 * lane) * 2);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + 64 * k));
    w[4 * k] = v.x;
    w[4 * k + 1] = v.y;
    w[4 * k + 2] = v.z;
    w[4 * k + 3] = v.w;
  }
}

// Loads the 32 elements of this lane's chunk (first element elem0, all of them < n) into w
// with 16-byte loads.
template <int DT>
__device__ __forceinline__ void load_chunk_full(const uint8_t* __restrict__ in, int64_t elem0, uint32_t* w) {
  const uint4* src = reinterpret_cast<const uint4*>(in + elem0 * (DT == F32 ? 4 : 2));
#pragma unroll
  for (int i = 0; i < Traits<DT>::kWords / 4; ++i) {
    const uint4 v = src[i];
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
}

// Loads the 32 elements of this lane's chunk (first element elem0) into w with 16-byte loads;
// returns how many are < n.  The ragged end loads element by element; elements past n read
// as NaN, which the absmax key excludes.
template <int DT>
__device__ __forceinline__ int load_chunk(const uint8_t* __restrict__ in, int64_t n, int64_t elem0, uint32_t* w) {
  using Tr = Traits<DT>;
  if (elem0 + kEPT <= n) {
    load_chunk_full<DT>(in, elem0, w);
    return 32;
  }
  const int nvalid = elem0 < n ? (int)(n - elem0) : 0;
#pragma unroll
  for (int i = 0; i < Tr::kWords; ++i) w[i] = Tr::kNaNWord;
  if constexpr (DT == F32) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(in) + elem0;
#pragma unroll
    for (int e = 0; e < 32; ++e)
      if (e < nvalid) w[e] = src[e];
  } else {
    // Every element is loaded into its own register first and the words are joined after by
    // byte permutes: merging each load into its word as it arrives (or shifting it in the
    // load's branch) made every load wait for the previous one.
    const unsigned short* src = reinterpret_cast<const unsigned short*>(in) + elem0;
    uint32_t h[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) h[e] = e < nvalid ? (uint32_t)src[e] : (Tr::kNaNWord & 0xffffu);
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = __builtin_amdgcn_perm(h[2 * i + 1], h[2 * i], 0x05040100u);
  }
  return nvalid;
}

// The lane's 32 elements of a full wave, loaded through LDS: the wave reads its 2048 elements
// as C rows of 64 x 16 bytes (one contiguous KiB per instruction, non-temporal: the input is
// read once), stores the 16-byte chunks in element order and each lane reads back its own C
// consecutive chunks.  Chunk q sits in slot q + q / C, which keeps the 16 lanes of every LDS
// access phase on distinct banks for both the writes and the reads.  With per-lane
// contiguous 16-byte loads straight from memory the kernel ran 7% slower on MI355X.
template <int DT>
struct LdsChunks {
  static constexpr int C = DT == F32 ? 8 : 4;  // 16-byte chunks per lane
  u32x4 t[C];
};

template <int DT>
__device__ __forceinline__ LdsChunks<DT> load_chunk_lds_issue(const uint8_t* __restrict__ in, int64_t wave0,
                                                               int lane) {
  LdsChunks<DT> r;
  const u32x4* src = reinterpret_cast<const u32x4*>(in + wave0 * (DT == F32 ? 4 : 2)) + lane;
#pragma unroll
  for (int c = 0; c < LdsChunks<DT>::C; ++c) r.t[c] = __builtin_nontemporal_load(src + c * 64);
  return r;
}

template <int DT>
__device__ __forceinline__ void load_chunk_lds_complete(const LdsChunks<DT>& r, int lane, uint4* tr, uint32_t* w) {
  constexpr int C = LdsChunks<DT>::C;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int q = c * 64 + lane;
    tr[q + q / C] = make_uint4(r.t[c].x, r.t[c].y, r.t[c].z, r.t[c].w);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int q = lane * C + i;
    const uint4 x = tr[q + q / C];
    w[4 * i] = x.x;
    w[4 * i + 1] = x.y;
    w[4 * i + 2] = x.z;
    w[4 * i + 3] = x.w;
  }
  __builtin_amdgcn_wave_barrier();  // later writes to tr come after these reads
}

// The lane's 32 elements of a full wave, loaded through LDS: the wave reads its 2048 elements
// as C rows of 64 x 16 bytes (one contiguous KiB per instruction, non-temporal: the input is
// read once), stores the 16-byte chunks in element order and each lane reads back its own C
// consecutive chunks.  Chunk q sits in slot q + q / C, which keeps the 16 lanes of every LDS
// access phase on distinct banks for both the writes and the reads.  With per-lane
// contiguous 16-byte loads straight from memory the kernel ran 7% slower on MI355X.  The
// loads are issued and completed by separate calls, so that other work can run between.
template <int DT>
__device__ __forceinline__ void load_chunk_lds(const uint8_t* __restrict__ in, int64_t wave0, int lane,
                                               uint4* tr, uint32_t* w) {
  load_chunk_lds_complete<DT>(load_chunk_lds_issue<DT>(in, wave0, lane), lane, tr, w);
}

struct QuantShared {
  uint32_t red[kThreads / 64];  // B = 4096: the two waves of a block exchange their keys
};

// Quantizes one lane chunk: block absmax, normalization, codes, packing and stores.  NESTED
// (the data pass of a nested quantize) stores the block maxima in the input's own format
// (binary32 for fp32 input, the 16 bits of fp16 / bf16 input, which hold them exactly);
// otherwise they are binary32.
template <int DT, int KB, int MODE, int M, bool NESTED, bool IL = false>
__device__ __forceinline__ void quantize_chunk(const uint32_t* w, int nvalid, int64_t elem0, int64_t n, int log2g,
                                               void* __restrict__ absmax, uint8_t* __restrict__ packed,
                                               const QuantArgs& qa, const typename Entry<M>::type* s_lut,
                                               const float* s_thr, QuantShared& sh, uint4* stage) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int G = 1 << log2g;
  const int64_t nb = (n + (kEPT << log2g) - 1) >> (5 + log2g);

  // Block absmax over G lanes.
  bool finite;
  uint32_t key = chunk_key<DT>(w, &finite);
  // Blocks of a whole wave or more (B >= 2048): DPP steps and lane reads, no LDS round trips.
  // Smaller blocks: LDS shuffles (the DPP form of group_max_u32, with its steps chosen at run
  // time, measured slower here: 2^29 bf16 4-bit 221.1 against 218.5 us).
  if (G >= 64) {
    key = wave_max_u32(key);
  } else {
    for (int m = 1; m < G; m <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, m));
  }
  if (G > 64) {  // B = 4096: two waves per block
    if (lane == 0) sh.red[tid >> 6] = key;
    __syncthreads();
    key = max(sh.red[tid >> 6], sh.red[(tid >> 6) ^ 1]);
    __syncthreads();
  }
  const float a = key_to_absmax<DT>(key);
  const int64_t blk = elem0 >> (5 + log2g);
  if ((tid & (G - 1)) == 0 && blk < nb) {
    if (NESTED && DT != F32)
      static_cast<uint16_t*>(absmax)[blk] = (uint16_t)key_to_bits16<DT>(key);
    else
      static_cast<float*>(absmax)[blk] = a;
  }

  // Normalize with the power-of-two guard; codes are packed into their output word as soon
  // as they are found (first element of a pair in the high nibble for 4-bit codes).
  const float s = a < 0x1p-64f ? 0x1p64f : (a > 0x1p64f ? 0x1p-64f : 1.0f);
  const float r = 1.0f / (a * s);
  constexpr int kOut = KB == 4 ? 4 : 8;  // output words per lane chunk
  constexpr int kPer = 32 / kOut;        // codes per output word
  uint32_t o[kOut];
  if (__builtin_expect(__all(finite && s == 1.0f && a > 0.0f), 1)) {
    // Every element of the wave is finite and every block maximum is nonzero and needs no
    // scaling: y = fl32(x * r) lies in [-1, 1] as it is.
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
      uint32_t q[kPer];
#pragma unroll
      for (int j = 0; j < kPer; j += 2)
        nearest_pair<MODE, M>(widen<DT>(w, i * kPer + j) * r, widen<DT>(w, i * kPer + j + 1) * r, qa, s_lut, s_thr,
                              q[j], q[j + 1]);
      o[i] = pack_word<KB>(q);
    }
  } else {
    // y = fl32(fl32(x * s) * r) for finite x in a block whose maximum is nonzero; a non-finite
    // x, and every element of a zero block, takes y = 0, whose code is z (the nearest code to
    // 0.0).  (Past n, the chunk holds NaN: code z, masked to the zero pad below.)  One element
    // at a time: taking pairs here as the fast path does doubled the kernel's registers.
    const bool live = a > 0.0f;
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
      uint32_t q[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const float x = widen<DT>(w, i * kPer + j);
        const float y = (x * s) * r;
        q[j] = nearest_code<MODE, M>(live && fabsf(x) <= 0x1.fffffep127f ? y : 0.0f, qa, s_lut, s_thr);
      }
      o[i] = pack_word<KB>(q);
    }
  }
  // codes of elements past n are 0 (the pad nibble of an odd n); wave-uniform test, so full
  // waves skip the masks instead of computing them
  if (__builtin_expect(!__all(nvalid >= 32), 0)) {
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
      const int c = min(max(nvalid - i * kPer, 0), kPer);
      uint32_t mask;
      if (KB == 4)
        mask = c >= 8 ? 0xffffffffu : ((1u << (8 * (c >> 1))) - 1u) | ((c & 1) ? (0xf0u << (8 * (c >> 1))) : 0u);
      else
        mask = c >= 4 ? 0xffffffffu : (1u << (8 * c)) - 1u;
      o[i] &= mask;
    }
  }

  // Store.  4-bit: each lane's 16 bytes follow its left neighbour's.  8-bit: a lane holds 32
  // bytes, so a wave's 2 KB goes through its 1 KB LDS region in two halves and leaves as two
  // 1 KB stores with consecutive lanes writing consecutive 16 bytes (in half h, lane l writes
  // half l & 1 of lane 32h + l/2).
  const int64_t packed_bytes = KB == 4 ? (n + 1) / 2 : n;
  constexpr int kBytes = kOut * 4;
  const int64_t off = KB == 4 ? elem0 >> 1 : elem0;
  const int64_t wave_off = off - (int64_t)lane * kBytes;
  if (IL) {  // interleaved chunk of a whole tile: word pair 2k holds segment k's 8 codes
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x2 v = {o[(2 * k) % kOut], o[(2 * k + 1) % kOut]};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(packed + wave_off + 512 * k + 8 * lane));
    }
  } else if (KB == 8 && wave_off + 64 * kBytes <= packed_bytes) {  // whole wave in range (uniform)
    // Two rounds through a 1 KB region: lanes 0-31, then 32-63, stage their bytes and the
    // whole wave stores them.
    uint8_t* dst = packed + wave_off;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if ((lane >> 5) == h) {
        stage[2 * (lane & 31)] = make_uint4(o[0], o[1], o[2], o[3]);
        stage[2 * (lane & 31) + 1] = make_uint4(o[4 % kOut], o[5 % kOut], o[6 % kOut], o[7 % kOut]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      store16_nt(dst + 1024 * h + 16 * lane, stage[lane]);
      __builtin_amdgcn_wave_barrier();  // the next round's writes come after these reads
    }
  } else if (KB == 4 && off + kBytes <= packed_bytes) {
    store16_nt(packed + off, make_uint4(o[0], o[1], o[2], o[3]));
  } else if (KB == 8 && off + kBytes <= packed_bytes) {
    store16_nt(packed + off, make_uint4(o[0], o[1], o[2], o[3]));
    store16_nt(packed + off + 16, make_uint4(o[4 % kOut], o[5 % kOut], o[6 % kOut], o[7 % kOut]));
  } else if (off < packed_bytes) {
#pragma unroll
    for (int i = 0; i < kBytes; ++i)
      if (off + i < packed_bytes) packed[off + i] = (uint8_t)(o[i >> 2] >> (8 * (i & 3)));
  }
}

// A workgroup quantizes one tile of 8192 elements, tile blockIdx.x.
template <int DT, int KB, int MODE, int M, bool NESTED>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const uint8_t* __restrict__ in, int64_t n, int log2g,
                                                            void* __restrict__ absmax,
                                                            uint8_t* __restrict__ packed, QuantArgs qa) {
  using Tr = Traits<DT>;
  using E = typename Entry<M>::type;
  __shared__ float s_thr[260];
  __shared__ E s_lut[LutLayout<MODE, M>::kSize];
  __shared__ uint4 s_stage[KB == 8 ? kThreads : 1];  // 8-bit codes: store exchange, 1 KB per wave
  __shared__ QuantShared sh;

  const int tid = threadIdx.x;
  const int64_t tile0 = blockIdx.x;
  // 4-bit codes load through LDS (see load_chunk_lds); 8-bit codes, whose LUT fills most of
  // the LDS, load directly.
  constexpr bool kViaLds = KB == 4;
  constexpr int kTrChunks = DT == F32 ? 576 : 320;  // padded chunk slots per wave
  __shared__ uint4 s_tr[kViaLds ? kThreads / 64 * kTrChunks : 1];
  uint4* tr = s_tr + (kViaLds ? (tid >> 6) * kTrChunks : 0);
  uint4* stage = s_stage + (KB == 8 ? (tid >> 6) * 64 : 0);
  const int64_t elem0 = (tile0 * kThreads + tid) * kEPT;
  uint32_t w[Tr::kWords];
  // The table words are loaded first, then the tile, and the LUT is filled while the tile is
  // in flight.  A complete tile (every tile but a partial last one; the test is uniform) takes
  // a path of unconditional loads of its own: where a load under a condition joins a path
  // without it, the compiler can only wait for every outstanding load, the tile's included,
  // before the LUT fill.
  constexpr bool kCanIL = KB == 8 && DT != F32;
  if (kCanIL && log2g >= 6 && (tile0 + 1) * kTile <= n) {  // uniform
    const auto lw = lut_fetch<MODE, M, kThreads>(qa, tid);
    load_chunk_il<DT>(in, elem0 - (int64_t)(tid & 63) * kEPT, tid & 63, w);
    lut_fill<MODE, M, kThreads>(qa, lw, s_lut, s_thr, tid);
    quantize_chunk<DT, KB, MODE, M, NESTED, kCanIL>(w, kEPT, elem0, n, log2g, absmax, packed, qa, s_lut, s_thr, sh,
                                                    stage);
  } else if ((tile0 + 1) * kTile <= n) {
    const auto lw = lut_fetch<MODE, M, kThreads>(qa, tid);
    if constexpr (kViaLds) {
      const auto chunks = load_chunk_lds_issue<DT>(in, elem0 - (int64_t)(tid & 63) * kEPT, tid & 63);
      lut_fill<MODE, M, kThreads>(qa, lw, s_lut, s_thr, tid);
      load_chunk_lds_complete<DT>(chunks, tid & 63, tr, w);
    } else {
      load_chunk_full<DT>(in, elem0, w);
      lut_fill<MODE, M, kThreads>(qa, lw, s_lut, s_thr, tid);
    }
    quantize_chunk<DT, KB, MODE, M, NESTED>(w, kEPT, elem0, n, log2g, absmax, packed, qa, s_lut, s_thr, sh,
                                            stage);
  } else {
    const auto lw = lut_fetch<MODE, M, kThreads>(qa, tid);
    const int64_t wave0 = elem0 - (int64_t)(tid & 63) * kEPT;
    int nvalid;
    if (kViaLds && wave0 + 64 * kEPT <= n) {  // uniform: the whole wave is in range
      load_chunk_lds<DT>(in, wave0, tid & 63, tr, w);
      nvalid = kEPT;
    } else {
      nvalid = load_chunk<DT>(in, n, elem0, w);
    }
    lut_fill<MODE, M, kThreads>(qa, lw, s_lut, s_thr, tid);
    quantize_chunk<DT, KB, MODE, M, NESTED>(w, nvalid, elem0, n, log2g, absmax, packed, qa, s_lut, s_thr, sh,
                                            stage);
  }
}

template <int DT, int KB, int MODE, int M>
hipError_t launch4(const void* in, int64_t n, int log2g, void* absmax, uint8_t* packed, bool nested,
                   const QuantArgs& qa, hipStream_t stream) {
  const dim3 grid((unsigned)quantize_grid(n));
  if (nested)
    return launch_kernel(quantize_kernel<DT, KB, MODE, M, true>, grid, dim3(kThreads), stream,
                         static_cast<const uint8_t*>(in), n, log2g, absmax, packed, qa);
  return launch_kernel(quantize_kernel<DT, KB, MODE, M, false>, grid, dim3(kThreads), stream,
                       static_cast<const uint8_t*>(in), n, log2g, absmax, packed, qa);
}

template <int DT, int KB>
hipError_t launch_mode(const void* in, int64_t n, int log2g, void* absmax, uint8_t* packed, bool nested,
                       const PreparedTable& t, hipStream_t s) {
  if (t.mode == LIN) {
    if (t.M <= 1) return launch4<DT, KB, LIN, 1>(in, n, log2g, absmax, packed, nested, t.qa, s);
    if (t.M == 2) return launch4<DT, KB, LIN, 2>(in, n, log2g, absmax, packed, nested, t.qa, s);
    return launch4<DT, KB, LIN, 3>(in, n, log2g, absmax, packed, nested, t.qa, s);
  }
  if (t.mode == F16B) return launch4<DT, KB, F16B, 1>(in, n, log2g, absmax, packed, nested, t.qa, s);
  if (t.mode == LOG) {
    if (t.M <= 1) return launch4<DT, KB, LOG, 1>(in, n, log2g, absmax, packed, nested, t.qa, s);
    if (t.M == 2) return launch4<DT, KB, LOG, 2>(in, n, log2g, absmax, packed, nested, t.qa, s);
    return launch4<DT, KB, LOG, 3>(in, n, log2g, absmax, packed, nested, t.qa, s);
  }
  return launch4<DT, KB, SEARCH, 1>(in, n, log2g, absmax, packed, nested, t.qa, s);
}

template <int DT>
hipError_t launch_dt(const void* in, int64_t n, int log2g, void* absmax, uint8_t* packed, bool nested,
                     const PreparedTable& t, hipStream_t s) {
  return t.K == 16 ? launch_mode<DT, 4>(in, n, log2g, absmax, packed, nested, t, s)
                   : launch_mode<DT, 8>(in, n, log2g, absmax, packed, nested, t, s);
}

}  // namespace

int quantize_grid(int64_t n) { return (int)((n + kTile - 1) / kTile); }

int launch_quantize(const void* in, int dtype, int64_t n, int blocksize, const PreparedTable& t, void* absmax,
                    uint8_t* packed, bool nested, void* stream) {
  int log2g = 0;
  while ((kEPT << log2g) < blocksize) ++log2g;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == F32) e = launch_dt<F32>(in, n, log2g, absmax, packed, nested, t, s);
  else if (dtype == F16) e = launch_dt<F16>(in, n, log2g, absmax, packed, nested, t, s);
  else e = launch_dt<BF16>(in, n, log2g, absmax, packed, nested, t, s);
  return (int)e;
}

}  // namespace bq
