// k_nested.hip -- second-level statistics of nested quantization (nested General8 /
// compressed-statistics NF4 of "Respect the current CUDA stream in blockwise quantization",
// bitsandbytes PR 2052, "Reproduced failure").
//
//   S     = binary64 pairwise sum of a_0..a_{nb-1}, zero-padded to a power-of-two length
//   mean  = RN32(S / nb)
//   d_b   = fl32(a_b - mean);  per group of B2 blocks: a2_g = max |d_b|,
//   q2_b  = nearest code of fl32(fl32(d_b * s) * fl32(1 / fl32(a2_g * s))) in the 256 table
//
// The data quantize kernel writes the block maxima (binary32, or the 16 bits of fp16 / bf16
// input, which hold them exactly).  Then:
//   run_sum_kernel: one workgroup per run of 16384 blocks sums the run's maxima as an aligned
//                   subtree of the mean's tree (blocks past nb count as +0, and x + 0 = x, so
//                   padding never changes a sum) into one binary64 run sum;
//   mean_kernel:    finishes the tree over the run sums (only when more than 512 remain);
//   stats_kernel:   finishes the tree itself otherwise (each workgroup, the same bits), then
//                   takes the same absmax / guard / LUT search as the data kernel over groups
//                   of the block maxima and writes q2 and the group maxima.
#include <hip/hip_runtime.h>

#include "bq_device.h"
#include "bq_launch.h"

namespace bq {
namespace {

constexpr int kMeanThreads = 1024;
constexpr int kLeaves = 32;                 // sums per lane
constexpr int kWaveLeaves = 64 * kLeaves;   // 2048: leaves per wave
constexpr int kChunk = 16 * kWaveLeaves;    // 32768: leaves per pass of mean_kernel

// Lane l of a wave adds leaves [32l, 32l+32) of a 2048-leaf run as a 5-level tree in
// registers, and the xor butterfly adds aligned runs of 32, 64, .., 2048 leaves (a + b and
// b + a round alike, so every lane ends with the same value).  Leaves at or past `count`
// read as +0, which leaves every sum unchanged.
__device__ __forceinline__ double wave_tree(const double* __restrict__ leaves, int64_t stride, int64_t i0,
                                            int64_t count, int lane) {
  const int64_t j0 = i0 + (int64_t)lane * kLeaves;
  double v[kLeaves];
  if (stride == 1 && j0 + kLeaves <= count) {
    const double2* p = reinterpret_cast<const double2*>(leaves + j0);
#pragma unroll
    for (int i = 0; i < kLeaves / 2; ++i) {
      const double2 d = p[i];
      v[2 * i] = d.x;
      v[2 * i + 1] = d.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kLeaves; ++i) v[i] = (j0 + i < count) ? leaves[(j0 + i) * stride] : 0.0;
  }
#pragma unroll
  for (int width = kLeaves; width > 1; width >>= 1)
#pragma unroll
    for (int i = 0; i < width / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  double s = v[0];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s = s + __shfl_xor(s, m);
  return s;
}

// The same tree over at most 512 leaves leaves[i * stride] (lane l adds leaves [8l, 8l+8) as
// a 3-level tree; the butterfly adds aligned runs of 8 .. 512), with a quarter of the registers.
__device__ __forceinline__ double wave_tree512(const double* __restrict__ leaves, int64_t stride, int64_t count,
                                               int lane) {
  double v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t j = (int64_t)lane * 8 + i;
    v[i] = j < count ? leaves[j * stride] : 0.0;
  }
#pragma unroll
  for (int width = 8; width > 1; width >>= 1)
#pragma unroll
    for (int i = 0; i < width / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  double s = v[0];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s = s + __shfl_xor(s, m);
  return s;
}
constexpr int64_t kFusedLeaves = 512;  // leaves the statistics kernel sums itself

// Block maxima as the data pass stores them: binary32, or the 16 bits of bf16 / fp16 input.
enum AbsmaxStore : int { AS_F32 = 0, AS_BF16 = 1, AS_F16 = 2 };

// Block maximum as binary32 from its stored bits.
template <int AS>
__device__ __forceinline__ float stored_absmax(uint32_t bits16_or_32) {
  if constexpr (AS == AS_F32) return bits_f32(bits16_or_32);
  else if constexpr (AS == AS_BF16) return bits_f32(bits16_or_32 << 16);
  else return (float)__builtin_bit_cast(_Float16, (unsigned short)bits16_or_32);
}

// First level of the mean's tree: workgroup r sums the maxima of blocks [16384r, 16384r +
// 16384) into runs[r].  Thread t adds its 64 blocks [64t, 64t + 64) of the run as a 6-level
// tree (eight 8-leaf trees, then a tree of their sums), the xor butterfly joins the aligned
// runs of 128 .. 4096 blocks inside each wave, and thread 0 joins the four waves as
// (w0 + w1) + (w2 + w3).  Every sum is an aligned subtree of the pairwise tree.
constexpr int kRunThreads = 256;
constexpr int kRunPerThread = (int)(kRunBlocks / kRunThreads);  // 64
static_assert(kRunPerThread == 64, "a thread sums 64 blocks");

template <int AS>
__global__ __launch_bounds__(kRunThreads) void run_sum_kernel(const void* __restrict__ absmax, int64_t nb,
                                                              double* __restrict__ runs) {
  __shared__ double s_w[kRunThreads / 64];
  const int t = threadIdx.x;
  const int64_t b0 = (int64_t)blockIdx.x * kRunBlocks + (int64_t)t * kRunPerThread;
  constexpr int kBytes = AS == AS_F32 ? 4 : 2;
  constexpr int kVec = kRunPerThread * kBytes / 16;  // 16-byte loads per thread
  uint32_t raw[kRunPerThread * kBytes / 4];
  const uint8_t* src = static_cast<const uint8_t*>(absmax) + b0 * kBytes;
  if (b0 + kRunPerThread <= nb) {
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(src)[i];
      raw[4 * i] = v.x;
      raw[4 * i + 1] = v.y;
      raw[4 * i + 2] = v.z;
      raw[4 * i + 3] = v.w;
    }
  } else {
    const int nv = b0 < nb ? (int)(nb - b0) : 0;
#pragma unroll
    for (int i = 0; i < kRunPerThread * kBytes / 4; ++i) raw[i] = 0u;
    if constexpr (AS == AS_F32) {
      for (int i = 0; i < nv; ++i) raw[i] = reinterpret_cast<const uint32_t*>(src)[i];
    } else {
      const uint16_t* h = reinterpret_cast<const uint16_t*>(src);
      for (int i = 0; i < nv; ++i) raw[i >> 1] |= (uint32_t)h[i] << (16 * (i & 1));
    }
  }
  double s8[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    double v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 8 * c + i;
      const uint32_t bits = AS == AS_F32 ? raw[k] : (raw[k >> 1] >> (16 * (k & 1))) & 0xffffu;
      v[i] = (double)stored_absmax<AS>(bits);
    }
    s8[c] = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
  }
  double s = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s = s + __shfl_xor(s, m);
  if ((t & 63) == 0) s_w[t >> 6] = s;
  __syncthreads();
  if (t == 0) runs[blockIdx.x] = (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]);
}

// Sum of `count` leaves leaves[i * stride]: 16 waves add a 32768-leaf chunk (wave sums
// joined as a 4-level tree by thread 0), and a binary counter in LDS joins the chunks (zero
// chunks pad the count to a power of two; they leave every sum unchanged).  mean = RN32(S / nb).
__global__ __launch_bounds__(kMeanThreads) void mean_kernel(const double* __restrict__ leaves, int64_t stride,
                                                            int64_t count, int64_t nb, float* __restrict__ mean) {
  __shared__ double s_w[kMeanThreads / 64];
  __shared__ double s_stack[40];
  __shared__ int s_has[40];
  const int t = threadIdx.x;
  if (t < 40) s_has[t] = 0;
  const int64_t nchunks = (count + kChunk - 1) / kChunk;
  for (int64_t c = 0; c < nchunks; ++c) {
    const double s = wave_tree(leaves, stride, c * kChunk + (int64_t)(t >> 6) * kWaveLeaves, count, t & 63);
    if ((t & 63) == 0) s_w[t >> 6] = s;
    __syncthreads();
    if (t == 0) {
      double w[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = s_w[i];
#pragma unroll
      for (int width = 16; width > 1; width >>= 1)
#pragma unroll
        for (int i = 0; i < width / 2; ++i) w[i] = w[2 * i] + w[2 * i + 1];
      double cs = w[0];
      int lvl = 0;
      for (int64_t k = c; k & 1; k >>= 1, ++lvl) {
        cs = s_stack[lvl] + cs;
        s_has[lvl] = 0;
      }
      s_stack[lvl] = cs;
      s_has[lvl] = 1;
    }
    __syncthreads();
  }
  if (t == 0) {
    // Pad with zero chunks: carry the lowest pending subtree upwards; a pending subtree at a
    // level is the left neighbour of everything below it.
    double carry = 0.0;
    bool any = false;
    for (int l = 0; l < 40; ++l) {
      if (s_has[l]) {
        carry = any ? s_stack[l] + carry : s_stack[l];
        any = true;
      }
    }
    *mean = (float)(carry / (double)nb);
  }
}

// Statistics of the groups.  A lane holds 16 consecutive blocks, so a group of B2 blocks is
// g = B2 / 16 consecutive lanes; a wave holds 1024 blocks and a workgroup of 4 waves a tile of
// 4096 (every group lies in one tile: B2 <= 4096).  The per-group work (maximum across lanes,
// guard, reciprocal) is one wave instruction for every group the wave holds at once, so with
// groups of 256 blocks it is shared by four groups.  Each workgroup takes kStatTiles
// consecutive tiles, loading the next tile while it codes the current one, and builds the LUT
// once for all of them.
constexpr int kStatThreads = 256;
constexpr int kBPL = 16;                           // blocks per lane
constexpr int kStatTile = kStatThreads * kBPL;     // 4096 blocks
constexpr int kStatTiles = 4;                      // tiles per workgroup

template <int AS>
struct AbsmaxLoad {
  static constexpr int kWords = AS == AS_F32 ? kBPL : kBPL / 2;  // 32-bit words per lane
  uint32_t w[kWords];
};

// Loads the lane's 16 block maxima of tile `tile` (raw words; blocks past nb read as zero).
template <int AS>
__device__ __forceinline__ AbsmaxLoad<AS> load_absmax(const void* __restrict__ absmax, int64_t nb, int64_t b0) {
  AbsmaxLoad<AS> r;
  constexpr int kW = AbsmaxLoad<AS>::kWords;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(absmax) +
                                                          b0 * (AS == AS_F32 ? 4 : 2));
  if (b0 + kBPL <= nb) {
    const uint4* p = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int i = 0; i < kW / 4; ++i) {
      const uint4 v = p[i];
      r.w[4 * i] = v.x;
      r.w[4 * i + 1] = v.y;
      r.w[4 * i + 2] = v.z;
      r.w[4 * i + 3] = v.w;
    }
  } else {
    const int nv = b0 < nb ? (int)(nb - b0) : 0;
    if constexpr (AS == AS_F32) {
#pragma unroll
      for (int i = 0; i < kW; ++i) r.w[i] = i < nv ? src[i] : 0u;
    } else {
      const uint16_t* h = reinterpret_cast<const uint16_t*>(src);
#pragma unroll
      for (int i = 0; i < kW; ++i) {
        const uint32_t lo = 2 * i < nv ? h[2 * i] : 0u;
        const uint32_t hi = 2 * i + 1 < nv ? h[2 * i + 1] : 0u;
        r.w[i] = lo | (hi << 16);
      }
    }
  }
  return r;
}

// Block maximum i of the lane (binary32).
template <int AS>
__device__ __forceinline__ float absmax_value(const AbsmaxLoad<AS>& r, int i) {
  if constexpr (AS == AS_F32) {
    return bits_f32(r.w[i]);
  } else if constexpr (AS == AS_BF16) {
    const uint32_t v = r.w[i >> 1];
    return bits_f32((i & 1) ? (v & 0xffff0000u) : (v << 16));
  } else {
    const uint32_t v = r.w[i >> 1];
    return (float)__builtin_bit_cast(_Float16, (unsigned short)((i & 1) ? (v >> 16) : (v & 0xffffu)));
  }
}

template <int AS, int MODE, int M>
__global__ __launch_bounds__(kStatThreads) void stats_kernel(const void* __restrict__ absmax, int64_t nb,
                                                             const double* __restrict__ leaves, int64_t stride,
                                                             int64_t count, float* __restrict__ mean, int log2b2,
                                                             int64_t ngroups, uint8_t* __restrict__ q2,
                                                             float* __restrict__ absmax2, QuantArgs qa) {
  using E = typename Entry<M>::type;
  __shared__ float s_thr[260];
  __shared__ E s_lut[LutLayout<MODE, M>::kSize];
  __shared__ float s_mean;
  __shared__ uint32_t s_red[2][kStatThreads / 64];  // groups wider than a wave: per-wave maxima
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = 1 << (log2b2 - 4);  // lanes per group (2 .. 256)
  const int64_t tile0 = (int64_t)blockIdx.x * kStatTiles;
  const int64_t ntiles = (nb + kStatTile - 1) / kStatTile;

  const auto lw = lut_fetch<MODE, M, kStatThreads>(qa, tid);  // table loads ahead of the data loads
  AbsmaxLoad<AS> cur = load_absmax<AS>(absmax, nb, tile0 * kStatTile + (int64_t)tid * kBPL);
  // With count > 0 every workgroup finishes the mean's tree itself (count <= 512 leaves, the
  // same bits in every workgroup); workgroup 0 stores it.  With count == 0 the mean is read.
  if (count > 0 && tid < 64) {
    const double S = wave_tree512(leaves, stride, count, tid);
    if (tid == 0) {
      const float mv = (float)(S / (double)nb);
      s_mean = mv;
      if (blockIdx.x == 0) *mean = mv;
    }
  }
  lut_fill<MODE, M, kStatThreads>(qa, lw, s_lut, s_thr, tid);  // ends with a barrier: s_mean is visible
  const float m = count > 0 ? s_mean : *mean;

  for (int k = 0; k < kStatTiles; ++k) {
    const int64_t tile = tile0 + k;
    if (tile >= ntiles) break;  // uniform
    const int64_t b0 = tile * kStatTile + (int64_t)tid * kBPL;
    AbsmaxLoad<AS> next = cur;
    if (k + 1 < kStatTiles && tile + 1 < ntiles)  // uniform
      next = load_absmax<AS>(absmax, nb, b0 + kStatTile);
    const bool whole = tile * kStatTile + kStatTile <= nb;  // uniform

    // d = a - mean; blocks past nb contribute nothing to a group maximum (|d| of a zero pad is
    // not used: those blocks are masked below).
    float d[kBPL];
#pragma unroll
    for (int i = 0; i < kBPL; ++i) d[i] = absmax_value<AS>(cur, i) - m;
    float amax = 0.0f;
    if (whole) {
#pragma unroll
      for (int i = 0; i < kBPL; ++i) amax = fmaxf(amax, fabsf(d[i]));
    } else {
#pragma unroll
      for (int i = 0; i < kBPL; ++i)
        if (b0 + i < nb) amax = fmaxf(amax, fabsf(d[i]));
    }
    // Group maximum: |d| is finite and not negative, so its bits order like its value.
    uint32_t key = f32_bits(amax);
    key = group_max_u32(key, g < 64 ? g : 64);
    if (g > 64) {  // groups of 2048 or 4096 blocks span 2 or 4 waves
      const int wave = tid >> 6;
      if (lane == 0) s_red[k & 1][wave] = key;
      __syncthreads();
      const int w0 = wave & ~((g >> 6) - 1);
      for (int w = 0; w < (g >> 6); ++w) key = max(key, s_red[k & 1][w0 + w]);
    }
    const float a2 = bits_f32(key);
    const int64_t grp = b0 >> log2b2;
    if ((tid & (g - 1)) == 0 && grp < ngroups) absmax2[grp] = a2;
    const float s = a2 < 0x1p-64f ? 0x1p64f : (a2 > 0x1p64f ? 0x1p-64f : 1.0f);
    // a group whose d are all zero (a2 = 0) takes y = 0, code z, everywhere
    const float rc = a2 > 0.0f ? 1.0f / (a2 * s) : 0.0f;
    uint32_t w[kBPL / 4];
    if (__builtin_expect(__all(s == 1.0f), 1)) {
#pragma unroll
      for (int j = 0; j < kBPL / 4; ++j) {
        uint32_t q[4];
#pragma unroll
        for (int i = 0; i < 4; i += 2)
          nearest_pair<MODE, M>(d[4 * j + i] * rc, d[4 * j + i + 1] * rc, qa, s_lut, s_thr, q[i], q[i + 1]);
        w[j] = pack_word<8>(q);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kBPL / 4; ++j) {
        uint32_t q[4];
#pragma unroll
        for (int i = 0; i < 4; i += 2)
          nearest_pair<MODE, M>((d[4 * j + i] * s) * rc, (d[4 * j + i + 1] * s) * rc, qa, s_lut, s_thr, q[i],
                                q[i + 1]);
        w[j] = pack_word<8>(q);
      }
    }
    if (whole) {
      *reinterpret_cast<uint4*>(q2 + b0) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if (b0 < nb) {
#pragma unroll
      for (int i = 0; i < kBPL; ++i)
        if (b0 + i < nb) q2[b0 + i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
    }
    cur = next;
  }
}

template <int AS, int MODE, int M>
hipError_t launch_stats(const void* absmax, int64_t nb, const double* leaves, int64_t stride, int64_t count,
                        float* mean, int log2b2, int64_t ngroups, uint8_t* q2, float* absmax2, const QuantArgs& qa,
                        hipStream_t s) {
  const int64_t per = (int64_t)kStatTile * kStatTiles;
  const dim3 grid((unsigned)((nb + per - 1) / per));
  return launch_kernel(stats_kernel<AS, MODE, M>, grid, dim3(kStatThreads), s, absmax, nb, leaves, stride, count,
                       mean, log2b2, ngroups, q2, absmax2, qa);
}

template <int AS>
hipError_t launch_stats_as(const void* absmax, int64_t nb, const double* leaves, int64_t stride, int64_t count,
                           float* mean, int log2b2, int64_t ngroups, uint8_t* q2, float* absmax2,
                           const PreparedTable& t2, hipStream_t s) {
  const QuantArgs& qa = t2.qa;
  if (t2.mode == LIN) {
    if (t2.M <= 1) return launch_stats<AS, LIN, 1>(absmax, nb, leaves, stride, count, mean, log2b2, ngroups, q2, absmax2, qa, s);
    if (t2.M == 2) return launch_stats<AS, LIN, 2>(absmax, nb, leaves, stride, count, mean, log2b2, ngroups, q2, absmax2, qa, s);
    return launch_stats<AS, LIN, 3>(absmax, nb, leaves, stride, count, mean, log2b2, ngroups, q2, absmax2, qa, s);
  }
  if (t2.mode == F16B)
    return launch_stats<AS, F16B, 1>(absmax, nb, leaves, stride, count, mean, log2b2, ngroups, q2, absmax2, qa, s);
  if (t2.mode == LOG) {
    if (t2.M <= 1) return launch_stats<AS, LOG, 1>(absmax, nb, leaves, stride, count, mean, log2b2, ngroups, q2, absmax2, qa, s);
    if (t2.M == 2) return launch_stats<AS, LOG, 2>(absmax, nb, leaves, stride, count, mean, log2b2, ngroups, q2, absmax2, qa, s);
    return launch_stats<AS, LOG, 3>(absmax, nb, leaves, stride, count, mean, log2b2, ngroups, q2, absmax2, qa, s);
  }
  return launch_stats<AS, SEARCH, 1>(absmax, nb, leaves, stride, count, mean, log2b2, ngroups, q2, absmax2, qa, s);
}

}  // namespace

int launch_nested_stats(const void* absmax, int dtype, int64_t nb, int blocksize2, const PreparedTable& t2,
                        double* runs, uint8_t* q2, float* absmax2, float* mean, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Run sums of 16384 blocks; up to 512 of them, the statistics kernel finishes the tree
  // itself; beyond (more than 2^23 blocks), mean_kernel does.
  const int64_t nruns = (nb + kRunBlocks - 1) / kRunBlocks;
  hipError_t e;
  const dim3 rgrid((unsigned)nruns);
  if (dtype == F32) e = launch_kernel(run_sum_kernel<AS_F32>, rgrid, dim3(kRunThreads), s, absmax, nb, runs);
  else if (dtype == BF16) e = launch_kernel(run_sum_kernel<AS_BF16>, rgrid, dim3(kRunThreads), s, absmax, nb, runs);
  else e = launch_kernel(run_sum_kernel<AS_F16>, rgrid, dim3(kRunThreads), s, absmax, nb, runs);
  if (e != hipSuccess) return (int)e;
  int64_t count = nruns;
  if (count > kFusedLeaves) {
    e = launch_kernel(mean_kernel, dim3(1), dim3(kMeanThreads), s, (const double*)runs, (int64_t)1, count, nb,
                      mean);
    if (e != hipSuccess) return (int)e;
    count = 0;
  }
  int log2b2 = 0;
  while ((1 << log2b2) < blocksize2) ++log2b2;
  const int64_t ngroups = (nb + blocksize2 - 1) / blocksize2;
  const double* leaves = runs;
  const int64_t stride = 1;
  if (dtype == F32)
    e = launch_stats_as<AS_F32>(absmax, nb, leaves, stride, count, mean, log2b2, ngroups, q2, absmax2, t2, s);
  else if (dtype == BF16)
    e = launch_stats_as<AS_BF16>(absmax, nb, leaves, stride, count, mean, log2b2, ngroups, q2, absmax2, t2, s);
  else
    e = launch_stats_as<AS_F16>(absmax, nb, leaves, stride, count, mean, log2b2, ngroups, q2, absmax2, t2, s);
  return (int)e;
}

}  // namespace bq
