// k_linear.hip -- fused dequantize + linear for small batches (decode) on gfx950:
// y = x . deq(W)^T, with W's dequantized values formed in registers and never written out
// (the weights-used-without-expanding approach of the mixed-input GEMMs in
// "stable-diffusion.cpp PR 2278", Summary, applied to the blockwise codes of this library).
//
//   W: N x K row-major, quantized blockwise over its flat index (element (n, k) is flat
//      element n*K + k), w = c[q] * a per element; x: M x K row-major, M <= 4.
//   y[m][n] = sum_k x[m][k] * c[q(n,k)] * a(n,k), accumulated in binary32.
//
// Work decomposition.  A workgroup owns 8 rows of W (4 when M > 2) and splits
// K among its 4 waves in chunks of 1024 (wave w takes chunks w, w + 4, ...).  A lane takes 16
// consecutive k of a chunk: it loads its x values once per chunk into registers and reuses
// them for those rows, whose codes (8 bytes for 4-bit, 16 for 8-bit: one load per lane and
// row, contiguous across the wave) all lie in one block, so the block scale multiplies the
// lane's 16-term partial sum once.  The HBM-bound stream is W's codes; x stays in L2.
// 4-bit codes go through a 256-entry LDS table of byte -> (c[high nibble], c[low nibble]),
// so one LDS read serves two elements.  At the end the rows x M sums of every lane and wave
// are transposed through LDS and added by all 256 threads.
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "bq_launch.h"

namespace bq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Rows of W per workgroup: 8 while the activations need few registers, 4 for M > 2 (measured
// at 14336 x 4096: 10.2 against 11.7 us for M = 1 with 8 rows; 17.4 against 18.7 us for M = 4
// with 4 rows).
template <int MT>
constexpr int rows_per_group() { return MT > 2 ? 4 : 8; }
constexpr int kLaneK = 16;  // consecutive k per lane and chunk (32 left half the waves idle at K = 4096: slower)
constexpr int kChunk = 64 * kLaneK;     // k per wave and chunk

// A lane's 16 activations of one row: the raw 16-byte words (loaded first, for every row,
// so that all loads are in flight together) and their binary32 values.
template <int DT>
struct XRaw {
  uint4 u[DT == F32 ? 4 : 2];
};

template <int DT>
__device__ __forceinline__ XRaw<DT> load_x16(const uint8_t* __restrict__ x, int64_t off) {
  XRaw<DT> r;
  const uint4* p = reinterpret_cast<const uint4*>(x + off * (DT == F32 ? 4 : 2));
#pragma unroll
  for (int i = 0; i < (DT == F32 ? 4 : 2); ++i) r.u[i] = p[i];
  return r;
}

template <int DT>
__device__ __forceinline__ void widen_x16(const XRaw<DT>& r, float* v) {
#pragma unroll
  for (int i = 0; i < (DT == F32 ? 4 : 2); ++i) {
    const uint32_t w[4] = {r.u[i].x, r.u[i].y, r.u[i].z, r.u[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (DT == F32) {
        v[4 * i + j] = __uint_as_float(w[j]);
      } else if constexpr (DT == BF16) {
        v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      } else {
        v[8 * i + 2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] & 0xffffu));
        v[8 * i + 2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] >> 16));
      }
    }
  }
}

// Codes of a lane's 16 elements of one row: 8 bytes (4-bit) or 16 bytes (8-bit).
template <int KB>
struct Codes {
  uint32_t w[KB == 4 ? 2 : 4];
};

template <int KB>
__device__ __forceinline__ Codes<KB> load_codes(const uint8_t* __restrict__ packed, int64_t flat) {
  Codes<KB> c;
  if constexpr (KB == 4) {
    const uint2 u = *reinterpret_cast<const uint2*>(packed + (flat >> 1));
    c.w[0] = u.x;
    c.w[1] = u.y;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(packed + flat);
    c.w[0] = u.x;
    c.w[1] = u.y;
    c.w[2] = u.z;
    c.w[3] = u.w;
  }
  return c;
}

// s[m] += sum over the lane's 16 elements of x[m][j] * c[q_j].
template <int KB, int MT>
__device__ __forceinline__ void dot16(const Codes<KB>& cd, const float (*xv)[kLaneK], const float2* s_pair,
                                      const float* s_c, float* s) {
#pragma unroll
  for (int b = 0; b < 8; ++b) {  // byte b of the 4-bit codes holds elements 2b (high) and 2b + 1
    float c0, c1;
    if constexpr (KB == 4) {
      const float2 p = s_pair[(cd.w[b >> 2] >> (8 * (b & 3))) & 0xffu];
      c0 = p.x;
      c1 = p.y;
    } else {
      c0 = s_c[(cd.w[b >> 1] >> (16 * (b & 1))) & 0xffu];
      c1 = s_c[(cd.w[b >> 1] >> (16 * (b & 1) + 8)) & 0xffu];
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      s[m] = __builtin_fmaf(xv[m][2 * b], c0, s[m]);
      s[m] = __builtin_fmaf(xv[m][2 * b + 1], c1, s[m]);
    }
  }
}

template <int DT, int KB, int MT>
__global__ __launch_bounds__(kThreads) void linear_kernel(const uint8_t* __restrict__ x, int M, int64_t K,
                                                          int64_t N, int log2b, const float* __restrict__ absmax,
                                                          const uint8_t* __restrict__ packed, float* __restrict__ y,
                                                          DequantArgs da) {
  constexpr int kRows = rows_per_group<MT>();
  __shared__ float2 s_pair[KB == 4 ? 256 : 1];
  __shared__ float s_c[KB == 8 ? 256 : 1];
  __shared__ float s_red[kRows * MT * kThreads];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if constexpr (KB == 4) s_pair[tid] = make_float2(da.c[tid >> 4], da.c[tid & 15]);
  else s_c[tid] = da.c[tid];
  __syncthreads();

  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t nchunks = (K + kChunk - 1) / kChunk;
  float acc[kRows][MT];
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  for (int64_t ch = wave; ch < nchunks; ch += kWaves) {
    const int64_t k0 = ch * kChunk + (int64_t)lane * kLaneK;
    if (k0 < K) {  // K is a multiple of 16: a lane's 16 elements are all inside or all outside
      // Every load is issued before any is used, with no branch around it: rows of W past N
      // and activation rows past M read a valid row instead, and their sums are never stored.
      Codes<KB> cd[kRows];
      float a[kRows];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int64_t flat = min(n0 + r, N - 1) * K + k0;
        cd[r] = load_codes<KB>(packed, flat);
        a[r] = absmax[flat >> log2b];
      }
      XRaw<DT> xr[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) xr[m] = load_x16<DT>(x, (int64_t)min(m, M - 1) * K + k0);
      float xv[MT][kLaneK];
#pragma unroll
      for (int m = 0; m < MT; ++m) widen_x16<DT>(xr[m], xv[m]);
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        float s[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) s[m] = 0.0f;
        dot16<KB, MT>(cd[r], xv, s_pair, s_c, s);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = __builtin_fmaf(a[r], s[m], acc[r][m]);
      }
    }
  }

  // Sums over the 256 threads: output o = r * MT + m sits at s_red[o * 256 + tid]; T threads
  // per output add 256 / T values each, then a shuffle tree joins the T partials.
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) s_red[(r * MT + m) * kThreads + tid] = acc[r][m];
  __syncthreads();
  constexpr int kOut = kRows * MT;
  constexpr int T = kThreads / kOut;  // 32, 16 or 16 threads per output
  const int o = tid / T;
  const int part = tid % T;
  float v = 0.0f;
#pragma unroll
  for (int i = 0; i < kThreads / T; ++i) v += s_red[o * kThreads + part * (kThreads / T) + i];
#pragma unroll
  for (int d = T / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  const int r = o / MT, m = o % MT;
  if (part == 0 && m < M && n0 + r < N) y[(int64_t)m * N + n0 + r] = v;
}

template <int DT, int KB>
hipError_t launch_mt(const void* x, int M, int64_t K, int64_t N, int log2b, const float* absmax,
                     const uint8_t* packed, float* y, const DequantArgs& da, hipStream_t s) {
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  auto grid = [N](int rows) { return dim3((unsigned)((N + rows - 1) / rows)); };
  if (M <= 1)
    return launch_kernel(linear_kernel<DT, KB, 1>, grid(rows_per_group<1>()), dim3(kThreads), s, xb, M, K, N, log2b, absmax, packed, y, da);
  if (M <= 2)
    return launch_kernel(linear_kernel<DT, KB, 2>, grid(rows_per_group<2>()), dim3(kThreads), s, xb, M, K, N, log2b, absmax, packed, y, da);
  return launch_kernel(linear_kernel<DT, KB, 4>, grid(rows_per_group<4>()), dim3(kThreads), s, xb, M, K, N, log2b, absmax, packed, y, da);
}

template <int DT>
hipError_t launch_kb(const void* x, int M, int64_t K, int64_t N, int log2b, const float* absmax,
                     const uint8_t* packed, float* y, const DequantArgs& da, hipStream_t s) {
  return da.K == 16 ? launch_mt<DT, 4>(x, M, K, N, log2b, absmax, packed, y, da, s)
                    : launch_mt<DT, 8>(x, M, K, N, log2b, absmax, packed, y, da, s);
}

}  // namespace

int launch_linear(const void* x, int dtype, int64_t M, int64_t K, int64_t N, int blocksize, const DequantArgs& da,
                  const float* absmax, const uint8_t* packed, float* y, void* stream) {
  int log2b = 0;
  while ((1 << log2b) < blocksize) ++log2b;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == F32) e = launch_kb<F32>(x, (int)M, K, N, log2b, absmax, packed, y, da, s);
  else if (dtype == F16) e = launch_kb<F16>(x, (int)M, K, N, log2b, absmax, packed, y, da, s);
  else e = launch_kb<BF16>(x, (int)M, K, N, log2b, absmax, packed, y, da, s);
  return (int)e;
}

}  // namespace bq
