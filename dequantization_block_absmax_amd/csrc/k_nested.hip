// k_nested.hip -- second-level statistics of nested quantization (nested General8 /
// compressed-statistics NF4 of "Respect the current CUDA stream in blockwise quantization",
// bitsandbytes PR 2052, "Reproduced failure").
//
//   S     = binary64 pairwise sum of a_0..a_{nb-1}, zero-padded to a power-of-two length
//   mean  = RN32(S / nb)
//   d_b   = fl32(a_b - mean);  per group of B2 blocks: a2_g = max |d_b|,
//   q2_b  = nearest code of fl32(fl32(d_b * s) * fl32(1 / fl32(a2_g * s))) in the 256 table
//
// The mean is a grid-wide dependency, so three kernels run in order on the stream:
//   partial_sums: one wave per aligned run of 256 leaves.  Lane l adds its 4 leaves as
//                 (a0 + a1) + (a2 + a3); xor-butterfly steps 1, 2, .., 32 then add aligned
//                 subtrees of 8, 16, .., 256 leaves: exactly the pairwise tree (binary64
//                 addition is commutative, so both partners compute the same bits).
//   mean:         one workgroup continues the same tree over the partial sums.
//   stats:        one wave per group; same absmax / guard / LUT search as the data kernel.
// Zero padding is exact inside the tree (x + 0 = x for x >= 0), so padding the 256-leaf runs
// and the partial sums to larger powers of two leaves S unchanged.
#include <hip/hip_runtime.h>

#include "bq_device.h"
#include "bq_launch.h"

namespace bq {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void partial_sums_kernel(const float* __restrict__ absmax, int64_t nb,
                                                                double* __restrict__ partials, int64_t nchunks) {
  const int lane = threadIdx.x & 63;
  const int64_t chunk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (chunk >= nchunks) return;  // whole waves exit together
  const int64_t i0 = chunk * 256 + lane * 4;
  double v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (i0 + i < nb) ? (double)absmax[i0 + i] : 0.0;
  double s = (v[0] + v[1]) + (v[2] + v[3]);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s = s + __shfl_xor(s, m);
  if (lane == 0) partials[chunk] = s;
}

// One workgroup of 1024 threads.  Thread t owns leaves [t*L, (t+1)*L) of the partial sums
// padded to 1024*L (L a power of two) and sums them pairwise with a binary-counter stack;
// then the wave butterfly and a 16-leaf tree over the waves finish the same tree.
__global__ __launch_bounds__(1024) void mean_kernel(const double* __restrict__ partials, int64_t nchunks,
                                                    int64_t L, int64_t nb, float* __restrict__ mean) {
  __shared__ double s_w[16];
  const int t = threadIdx.x;
  double stack[40];
  for (int64_t i = 0; i < L; ++i) {
    const int64_t leaf = (int64_t)t * L + i;
    double v = leaf < nchunks ? partials[leaf] : 0.0;
    int lvl = 0;
    for (int64_t k = i; k & 1; k >>= 1, ++lvl) v = stack[lvl] + v;
    stack[lvl] = v;
  }
  int top = 0;
  while ((int64_t(1) << top) < L) ++top;
  double s = stack[top];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s = s + __shfl_xor(s, m);
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
    *mean = (float)(w[0] / (double)nb);
  }
}

template <int MODE, int M>
__global__ __launch_bounds__(kThreads) void stats_kernel(const float* __restrict__ absmax, int64_t nb,
                                                         const float* __restrict__ mean, int log2b2,
                                                         int64_t ngroups, uint8_t* __restrict__ q2,
                                                         float* __restrict__ absmax2, QuantArgs qa) {
  using E = typename Entry<M>::type;
  __shared__ float s_thr[260];
  __shared__ E s_lut[MODE == SEARCH ? 1 : kLutMax];
  const int tid = threadIdx.x;
  build_lut<MODE, M>(qa, s_lut, s_thr, tid, kThreads);

  const int lane = tid & 63;
  const float m = *mean;
  const int B2 = 1 << log2b2;
  const int per = B2 >= 64 ? B2 / 64 : 1;
  for (int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + (tid >> 6); g < ngroups;
       g += (int64_t)gridDim.x * (kThreads / 64)) {
    const int64_t b0 = g << log2b2;
    uint32_t key = 0;  // |d| bit patterns; all d are finite
    for (int i = 0; i < per; ++i) {
      const int64_t v = i * 64 + lane;
      const int64_t b = b0 + v;
      if (v < B2 && b < nb) {
        const float d = absmax[b] - m;
        key = max(key, f32_bits(d) & 0x7fffffffu);
      }
    }
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, k));
    const float a2 = bits_f32(key);
    if (lane == 0) absmax2[g] = a2;
    const float s = a2 < 0x1p-64f ? 0x1p64f : (a2 > 0x1p64f ? 0x1p-64f : 1.0f);
    const float r = 1.0f / (a2 * s);
    for (int i = 0; i < per; ++i) {
      const int64_t v = i * 64 + lane;
      const int64_t b = b0 + v;
      if (v < B2 && b < nb) {
        const float d = absmax[b] - m;
        const float y = (s == 1.0f) ? d * r : (d * s) * r;
        q2[b] = (uint8_t)nearest_code<MODE, M>(y, qa, s_lut, s_thr);
      }
    }
  }
}

template <int MODE, int M>
hipError_t launch_stats(const float* absmax, int64_t nb, const float* mean, int log2b2, int64_t ngroups,
                        uint8_t* q2, float* absmax2, const QuantArgs& qa, hipStream_t s) {
  int64_t grid = (ngroups + 3) / 4;
  if (grid > 2048) grid = 2048;
  return launch_kernel(stats_kernel<MODE, M>, dim3((unsigned)grid), dim3(kThreads), s, absmax, nb, mean, log2b2,
                       ngroups, q2, absmax2, qa);
}

}  // namespace

int launch_nested_stats(const float* absmax, int64_t nb, int blocksize2, const PreparedTable& t2, double* partials,
                        uint8_t* q2, float* absmax2, float* mean, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nchunks = (nb + 255) / 256;
  hipError_t e = launch_kernel(partial_sums_kernel, dim3((unsigned)((nchunks + 3) / 4)), dim3(kThreads), s, absmax,
                               nb, partials, nchunks);
  if (e != hipSuccess) return (int)e;
  int64_t L = 1;
  while (L * 1024 < nchunks) L *= 2;
  e = launch_kernel(mean_kernel, dim3(1), dim3(1024), s, partials, nchunks, L, nb, mean);
  if (e != hipSuccess) return (int)e;
  int log2b2 = 0;
  while ((1 << log2b2) < blocksize2) ++log2b2;
  const int64_t ngroups = (nb + blocksize2 - 1) / blocksize2;
  const QuantArgs& qa = t2.qa;
  if (t2.mode == LIN) {
    if (t2.M <= 1) e = launch_stats<LIN, 1>(absmax, nb, mean, log2b2, ngroups, q2, absmax2, qa, s);
    else if (t2.M == 2) e = launch_stats<LIN, 2>(absmax, nb, mean, log2b2, ngroups, q2, absmax2, qa, s);
    else e = launch_stats<LIN, 3>(absmax, nb, mean, log2b2, ngroups, q2, absmax2, qa, s);
  } else if (t2.mode == LOG) {
    if (t2.M <= 1) e = launch_stats<LOG, 1>(absmax, nb, mean, log2b2, ngroups, q2, absmax2, qa, s);
    else if (t2.M == 2) e = launch_stats<LOG, 2>(absmax, nb, mean, log2b2, ngroups, q2, absmax2, qa, s);
    else e = launch_stats<LOG, 3>(absmax, nb, mean, log2b2, ngroups, q2, absmax2, qa, s);
  } else {
    e = launch_stats<SEARCH, 1>(absmax, nb, mean, log2b2, ngroups, q2, absmax2, qa, s);
  }
  return (int)e;
}

}  // namespace bq
