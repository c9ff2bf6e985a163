// k_nested.hip -- second-level statistics of nested quantization (nested General8 /
// compressed-statistics NF4 of "Respect the current CUDA stream in blockwise quantization",
// bitsandbytes PR 2052, "Reproduced failure").
//
//   S     = binary64 pairwise sum of a_0..a_{nb-1}, zero-padded to a power-of-two length
//   mean  = RN32(S / nb)
//   d_b   = fl32(a_b - mean);  per group of B2 blocks: a2_g = max |d_b|,
//   q2_b  = nearest code of fl32(fl32(d_b * s) * fl32(1 / fl32(a2_g * s))) in the 256 table
//
// The data quantize kernel already writes, per wave of 2048 elements, the pairwise sum of its
// blocks' maxima: an aligned subtree of 2^k leaves of the mean's tree (blocks past n hold +0, and
// x + 0 = x, so padding never changes a sum).  Then:
//   run_sum_kernel: sums runs of 2048 partials in place (more than 512 partials);
//   mean_kernel:    finishes the tree (only when more than 512 run sums remain);
//   stats_kernel:   finishes the tree itself otherwise (each workgroup, the same bits), then
//                   one wave per 1024, 2048 or 4096 blocks (4 consecutive per lane per run of 256)
//                   takes the same absmax / guard / LUT search as the data kernel and writes
//                   q2 and the group maxima.
#include <hip/hip_runtime.h>

#include "bq_device.h"
#include "bq_launch.h"

namespace bq {
namespace {

constexpr int kThreads = 512;  // statistics workgroup: eight waves share one LUT
constexpr int kWaves = kThreads / 64;
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

// First level over many per-wave partial sums: wave w replaces leaf 2048w by the sum of
// leaves [2048w, 2048w + 2048), an aligned subtree of the same tree (it reads its whole run
// before lane 0 writes, and no other wave reads that run).
__global__ __launch_bounds__(64) void run_sum_kernel(double* __restrict__ partials, int64_t npart) {
  const int64_t i0 = (int64_t)blockIdx.x * kWaveLeaves;
  const double s = wave_tree(partials, 1, i0, npart, threadIdx.x);
  if (threadIdx.x == 0) partials[i0] = s;
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

// One wave covers KR runs of 256 consecutive blocks (lane l holds blocks 4l..4l+3 of each run);
// a group of B2 blocks is ceil(B2 / 256) whole runs, or B2 / 4 lanes of one run.  All of a
// wave's loads are issued before the LUT prologue.
template <int MODE, int M, int KR, bool kRoundwise>
__global__ __launch_bounds__(kThreads) void stats_kernel(const float* __restrict__ absmax, int64_t nb,
                                                         const double* __restrict__ leaves, int64_t stride,
                                                         int64_t count, float* __restrict__ mean, int log2b2,
                                                         int64_t ngroups, uint8_t* __restrict__ q2,
                                                         float* __restrict__ absmax2, QuantArgs qa) {
  using E = typename Entry<M>::type;
  __shared__ float s_thr[260];
  __shared__ E s_lut[LutLayout<MODE, M>::kSize];
  __shared__ float s_mean;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int B2 = 1 << log2b2;
  const int R = B2 > 256 ? B2 >> 8 : 1;       // runs per group
  const int lg = B2 >= 256 ? 64 : (B2 >> 2);  // lanes per group inside a run
  const int64_t b0 = ((int64_t)blockIdx.x * kWaves + (tid >> 6)) * 256 * KR + lane * 4;
  const bool active = b0 - lane * 4 < nb;

  const auto lw = lut_fetch<MODE, M, kThreads>(qa, tid);  // table loads ahead of the data loads
  float4 v[KR];
#pragma unroll
  for (int r = 0; r < KR; ++r) {
    const int64_t b = b0 + r * 256;
    v[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (b + 4 <= nb) {
      v[r] = *reinterpret_cast<const float4*>(absmax + b);
    } else if (b < nb) {
      v[r].x = absmax[b];
      if (b + 1 < nb) v[r].y = absmax[b + 1];
      if (b + 2 < nb) v[r].z = absmax[b + 2];
    }
  }
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
  lut_fill<MODE, M, kThreads>(qa, lw, s_lut, s_thr, tid);  // ends with a barrier: s_mean is visible
  if (!active) return;  // whole waves
  const float m = count > 0 ? s_mean : *mean;

  // Codes and q2 of run r, given the group maximum key of its blocks.
  auto emit = [&](int r, uint32_t key, const float* d) {
    const int64_t b = b0 + r * 256;
    const float a2 = bits_f32(key);
    const int64_t g = b >> log2b2;
    if ((lane & (lg - 1)) == 0 && (r & (R - 1)) == 0 && g < ngroups) absmax2[g] = a2;
    const float s = a2 < 0x1p-64f ? 0x1p64f : (a2 > 0x1p64f ? 0x1p-64f : 1.0f);
    const float rc = 1.0f / (a2 * s);
    // (d * s) * rc is d * rc when s = 1; a wave-uniform test lets the common case skip the
    // scaling instead of computing both and selecting.
    uint32_t q[4];
    if (__builtin_expect(__all(s == 1.0f), 1)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = nearest_code<MODE, M>(d[i] * rc, qa, s_lut, s_thr);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = nearest_code<MODE, M>((d[i] * s) * rc, qa, s_lut, s_thr);
    }
    const uint32_t w = pack_word<8>(q);
    if (b + 4 <= nb) {
      *reinterpret_cast<uint32_t*>(q2 + b) = w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (b + i < nb) q2[b + i] = (uint8_t)(w >> (8 * i));
    }
  };

  // d = a - mean; blocks past nb contribute nothing to a group maximum.
  if constexpr (kRoundwise) {
    // B2 <= 256: every group lies inside one run, so each run is finished as soon as its
    // loads arrive, overlapping the codes of early runs with the loads of later ones.
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int64_t b = b0 + r * 256;
      const float d[4] = {v[r].x - m, v[r].y - m, v[r].z - m, v[r].w - m};
      uint32_t key = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (b + i < nb) key = max(key, f32_bits(d[i]) & 0x7fffffffu);
      key = group_max_u32(key, lg);
      if (b < nb) emit(r, key, d);
    }
  } else {
    uint32_t key[KR];
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int64_t b = b0 + r * 256;
      float d[4] = {v[r].x - m, v[r].y - m, v[r].z - m, v[r].w - m};
      key[r] = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (b + i < nb) key[r] = max(key[r], f32_bits(d[i]) & 0x7fffffffu);
      v[r] = make_float4(d[0], d[1], d[2], d[3]);
    }
#pragma unroll
    for (int r = 0; r < KR; ++r)
      key[r] = group_max_u32(key[r], lg);
    // groups of R runs: an xor butterfly over run indices gives every run its group's maximum
#pragma unroll
    for (int st = 1; st < KR; st <<= 1)
      if (st < R) {
#pragma unroll
        for (int r = 0; r < KR; ++r)
          if ((r & st) == 0) {
            const uint32_t k2 = max(key[r], key[r | st]);
            key[r] = k2;
            key[r | st] = k2;
          }
      }
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const float d[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
      if (b0 + r * 256 < nb) emit(r, key[r], d);
    }
  }
}

template <int MODE, int M>
hipError_t launch_stats(const float* absmax, int64_t nb, const double* leaves, int64_t stride, int64_t count,
                        float* mean, int log2b2, int64_t ngroups, uint8_t* q2, float* absmax2, const QuantArgs& qa,
                        hipStream_t s) {
  // runs per wave: a group (B2 / 256 runs) fits in a wave; groups inside a run take 4 runs per
  // wave (more waves in flight: 2^23 blocks, 245.6 against 249.1 us for the whole nested call)
  const int kr = log2b2 > 11 ? 16 : (log2b2 > 8 ? 8 : 4);
  const dim3 grid((unsigned)((nb + kWaves * 256 * kr - 1) / (kWaves * 256 * kr)));
  if (log2b2 > 11)
    return launch_kernel(stats_kernel<MODE, M, 16, false>, grid, dim3(kThreads), s, absmax, nb, leaves, stride,
                         count, mean, log2b2, ngroups, q2, absmax2, qa);
  if (log2b2 > 8)
    return launch_kernel(stats_kernel<MODE, M, 8, false>, grid, dim3(kThreads), s, absmax, nb, leaves, stride,
                         count, mean, log2b2, ngroups, q2, absmax2, qa);
  return launch_kernel(stats_kernel<MODE, M, 4, true>, grid, dim3(kThreads), s, absmax, nb, leaves, stride, count,
                       mean, log2b2, ngroups, q2, absmax2, qa);
}

}  // namespace

int launch_nested_stats(const float* absmax, int64_t nb, int blocksize2, const PreparedTable& t2,
                        double* partials, int64_t npart, uint8_t* q2, float* absmax2, float* mean,
                        void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Above 512 partial sums, runs of 2048 are first summed in place by one wave each (one
  // workgroup reading them all would be bound by a single CU's bandwidth).  Up to 512 leaves
  // remain, the statistics kernel finishes the tree itself; beyond, mean_kernel does.
  hipError_t e;
  double* leaves = partials;
  int64_t stride = 1, count = npart;
  if (npart > kFusedLeaves) {
    const int64_t runs = (npart + kWaveLeaves - 1) / kWaveLeaves;
    e = launch_kernel(run_sum_kernel, dim3((unsigned)runs), dim3(64), s, leaves, npart);
    if (e != hipSuccess) return (int)e;
    stride = kWaveLeaves;
    count = runs;
  }
  if (count > kFusedLeaves) {
    e = launch_kernel(mean_kernel, dim3(1), dim3(kMeanThreads), s, (const double*)leaves, stride, count, nb, mean);
    if (e != hipSuccess) return (int)e;
    count = 0;
  }
  int log2b2 = 0;
  while ((1 << log2b2) < blocksize2) ++log2b2;
  const int64_t ngroups = (nb + blocksize2 - 1) / blocksize2;
  const QuantArgs& qa = t2.qa;
  auto go = [&](auto kernel_launcher) {
    return kernel_launcher(absmax, nb, leaves, stride, count, mean, log2b2, ngroups, q2, absmax2, qa, s);
  };
  if (t2.mode == LIN) {
    if (t2.M <= 1) e = go(launch_stats<LIN, 1>);
    else if (t2.M == 2) e = go(launch_stats<LIN, 2>);
    else e = go(launch_stats<LIN, 3>);
  } else if (t2.mode == LOG) {
    if (t2.M <= 1) e = go(launch_stats<LOG, 1>);
    else if (t2.M == 2) e = go(launch_stats<LOG, 2>);
    else e = go(launch_stats<LOG, 3>);
  } else {
    e = go(launch_stats<SEARCH, 1>);
  }
  return (int)e;
}

}  // namespace bq
