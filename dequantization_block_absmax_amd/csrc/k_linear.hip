// k_linear.hip -- fused dequantize + linear for small batches (decode) on gfx950:
// y = x . deq(W)^T, with W's dequantized values formed in registers and never written out
// (the weights-used-without-expanding approach of the mixed-input GEMMs in
// "stable-diffusion.cpp PR 2278", Summary, applied to the blockwise codes of this library).
//
//   W: N x K row-major, quantized blockwise over its flat index (element (n, k) is flat
//      element n*K + k), w = c[q] * a per element; x: M x K row-major, M <= 4.
//   y[m][n] = sum_k x[m][k] * c[q(n,k)] * a(n,k), accumulated in binary32.
//
// Two forms.  The vector form below serves every shape; the matrix-core form further down
// serves tall weights with 4-bit codes at M = 3 or 4, where it measured faster.
//
// Vector form.  A workgroup owns 8 rows of W (4 when M > 2) and splits
// K among its 4 waves in chunks of 1024 (wave w takes chunks w, w + 4, ...).  A lane takes 16
// consecutive k of a chunk: it loads its x values once per chunk into registers and reuses
// them for those rows, whose codes (8 bytes for 4-bit, 16 for 8-bit: one load per lane and
// row, contiguous across the wave) all lie in one block, so the block scale multiplies the
// lane's 16-term partial sum once.  The HBM-bound stream is W's codes; x stays in L2.
// 4-bit codes go through a 256-entry LDS table of byte -> (c[high nibble], c[low nibble]),
// so one LDS read serves two elements.  At the end the rows x M sums of every lane and wave
// are transposed through LDS and added by all 256 threads.
#include <hip/hip_runtime.h>

#include <atomic>

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

// Codes of a lane's 16 elements of one row: 8 bytes (4-bit) or 16 bytes (8-bit), loaded
// non-temporally: each load instruction of a wave reads 512 or 1024 consecutive bytes of the
// row, whole cache lines, read once (1-5% faster at 14336 x 4096 and 4096 x 14336; 8-bit
// M = 4: 19.0 against 20.0 us).
template <int KB>
struct Codes {
  uint32_t w[KB == 4 ? 2 : 4];
};

template <int KB>
__device__ __forceinline__ Codes<KB> load_codes(const uint8_t* __restrict__ packed, int64_t flat) {
  Codes<KB> c;
  typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));
  typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
  if constexpr (KB == 4) {
    const u32x2_nt u = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(packed + (flat >> 1)));
    c.w[0] = u.x;
    c.w[1] = u.y;
  } else {
    const u32x4_nt u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(packed + flat));
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

// ---- Matrix-core form (4-bit codes, M = 3 or 4, tall weights) ----
//
// v_mfma_f32_4x4x1f32 performs 16 independent 4 x 4 outer-product updates per wave: lane l
// supplies A[i] and B[j] (i = j = l % 4) of instruction block l / 4 and holds D[v][l % 4] of
// that block in accumulator element v.  An in-bounds probe fixed this layout on MI355X and
// showed that each update rounds once, as an FMA, and keeps binary32 subnormals.  Instruction
// block b is lane block b of the wave, which walks the 64 k of one quantization block one k per
// step: lane 4b + i supplies x[i][k] as A and the code value c[q] of weight row n0 + i as B, so
// after 64 steps lane l holds, for row n0 + l % 4, the sums over its 64 k of x[m][k] c[q] for
// m = 0..3.  Each sum is a chain of binary32 FMAs, as in the vector form, but the four
// activation rows share each weight: one matrix instruction does the four FMAs of 64 weights,
// and the vector units are left with the code lookups.
//
// A workgroup has ceil(K / 1024) waves (K <= 4096); wave w owns k in [1024 w, 1024 w + 1024)
// (16 lane blocks of 64 k) and holds its lanes' 64 activations in registers for the whole
// launch.  It walks a run of up to 8 tiles of 4 weight rows, loading the next tile's codes and
// block maxima while the current one is multiplied.  Four accumulators take the steps in turn
// (16-term chains).  A tile's sums are scaled by their block maxima, added over the 16 lane
// blocks (two permlane swaps, two row rotations) and over the waves, in wave order, through LDS.
constexpr int kMfmaWaves = 4;
constexpr int kMfmaTiles = 8;  // tiles per workgroup (even: an odd run is padded with a repeat)

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct MTile {
  uint4 u[2];  // the lane's 64 four-bit codes of one row
  float a;     // their block maximum
};

__device__ __forceinline__ void load_mtile(MTile& t, const uint8_t* packed, const float* absmax, int64_t row,
                                           int64_t K, int64_t k0, int log2b) {
  const int64_t flat = row * K + k0;
  const uint4* p = reinterpret_cast<const uint4*>(packed + (flat >> 1));
  t.u[0] = p[0];
  t.u[1] = p[1];
  t.a = absmax[flat >> log2b];
}

__device__ __forceinline__ float2 swap_halves(float lo, float hi) {  // lanes 32-63 of lo <-> 0-31 of hi
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float2 swap_rows(float lo, float hi) {  // odd 16-lane rows of lo <-> even rows of hi
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int DT>
__global__ __launch_bounds__(64 * kMfmaWaves) void linear_mfma_kernel(
    const uint8_t* x, int M, int64_t K, int64_t N, int log2b, const float* absmax, const uint8_t* packed,
    float* __restrict__ y, DequantArgs da, int64_t ntiles) {
  __shared__ float2 s_pair[256];
  __shared__ float s_part[kMfmaTiles * kMfmaWaves * 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = blockDim.x >> 6;
  for (int i = tid; i < 256; i += blockDim.x) s_pair[i] = make_float2(da.c[i >> 4], da.c[i & 15]);

  // Lane 4b + i: activation row i, k from k0 = 1024 wave + 64 b.  Lane blocks past K read k = 0
  // and weigh it by zero (activations and block maximum 0; codes are finite), as do activation
  // rows past M.
  const int li = lane & 3;
  const int64_t kl = (int64_t)wave * kChunk + (int64_t)(lane >> 2) * 64;
  const bool live = kl < K;
  const int64_t k0 = live ? kl : 0;
  float xv[64];
  {
    const bool xlive = live && li < M;
    const int64_t off = (int64_t)min(li, M - 1) * K + k0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const XRaw<DT> r = load_x16<DT>(x, off + 16 * c);
      widen_x16<DT>(r, xv + 16 * c);
    }
#pragma unroll
    for (int j = 0; j < 64; ++j) xv[j] = xlive ? xv[j] : 0.0f;
  }
  const int64_t tile0 = (int64_t)blockIdx.x * kMfmaTiles;
  const int n = (int)min((int64_t)kMfmaTiles, ntiles - tile0);
  __syncthreads();  // the code table

  auto process = [&](const MTile& t, int i) {
    f32x4 acc[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t w[8] = {t.u[0].x, t.u[0].y, t.u[0].z, t.u[0].w, t.u[1].x, t.u[1].y, t.u[1].z, t.u[1].w};
#pragma unroll
    for (int b = 0; b < 32; ++b) {  // byte b holds k = 2b (high nibble) and 2b + 1
      const float2 c = s_pair[(w[b >> 2] >> (8 * (b & 3))) & 0xffu];
      acc[(2 * b) & 3] = __builtin_amdgcn_mfma_f32_4x4x1f32(xv[2 * b], c.x, acc[(2 * b) & 3], 0, 0, 0);
      acc[(2 * b + 1) & 3] = __builtin_amdgcn_mfma_f32_4x4x1f32(xv[2 * b + 1], c.y, acc[(2 * b + 1) & 3], 0, 0, 0);
    }
    const float a = live ? t.a : 0.0f;
    float v[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) v[m] = a * ((acc[0][m] + acc[1][m]) + (acc[2][m] + acc[3][m]));
    // Sum over the 16 lane blocks (lane bits 2..5).  A swap on lane bit 5, then one on bit 4,
    // each keeps half of the values (the lower half where the bit is clear) and adds the
    // partner's copy; two row rotations add over bits 3 and 2.  Lane l ends with row l % 4,
    // activation row l / 16.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float2 r = swap_halves(v[j], v[j + 2]);
      v[j] = r.x + r.y;
    }
    const float2 r = swap_rows(v[0], v[1]);
    float tot = r.x + r.y;
    tot += dpp<0x124>(tot);  // row_ror:4
    tot += dpp<0x128>(tot);  // row_ror:8
    if ((lane & 12) == 0) s_part[(i * kMfmaWaves + wave) * 16 + (lane >> 4) * 4 + li] = tot;
  };

  // Rows past N read row N - 1; their sums are never stored.
  auto row_of = [&](int i) { return min((tile0 + min(i, n - 1)) * 4 + li, N - 1); };
  MTile ta, tb;
  load_mtile(ta, packed, absmax, row_of(0), K, k0, log2b);
  for (int i = 0; i < n; i += 2) {
    load_mtile(tb, packed, absmax, row_of(i + 1), K, k0, log2b);
    __builtin_amdgcn_sched_barrier(0);
    process(ta, i);
    load_mtile(ta, packed, absmax, row_of(i + 2), K, k0, log2b);
    __builtin_amdgcn_sched_barrier(0);
    process(tb, i + 1);  // i + 1 == n only for an odd run: a repeat into a slot never read
  }
  __syncthreads();

  for (int o = tid; o < n * 16; o += blockDim.x) {
    const int i = o >> 4, ov = o & 15;
    float sum = 0.0f;
    for (int w = 0; w < nwaves; ++w) sum += s_part[(i * kMfmaWaves + w) * 16 + ov];
    const int64_t row = (tile0 + i) * 4 + (ov & 3);
    const int m = ov >> 2;
    if (m < M && row < N) y[(int64_t)m * N + row] = sum;
  }
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
  // The matrix-core form where it measured faster: 4-bit codes, M = 3 or 4, K <= 4096 (a
  // multiple of 64), blocks of at least 64 and at least 32 weight rows per CU.  At 14336 x 4096
  // it takes 13.3 us against 17.5 for M = 4; at 4096 rows it was no faster.
  if (KB == 4 && K % 64 == 0 && K <= kMfmaWaves * kChunk && log2b >= 6 && N >= 32 * (int64_t)cu_count()) {
    const int64_t ntiles = (N + 3) / 4;
    return launch_kernel(linear_mfma_kernel<DT>, dim3((unsigned)((ntiles + kMfmaTiles - 1) / kMfmaTiles)),
                         dim3((unsigned)(64 * ((K + kChunk - 1) / kChunk))), s, xb, M, K, N, log2b, absmax, packed,
                         y, da, ntiles);
  }
  return launch_kernel(linear_kernel<DT, KB, 4>, grid(rows_per_group<4>()), dim3(kThreads), s, xb, M, K, N, log2b, absmax, packed, y, da);
}

template <int DT>
hipError_t launch_kb(const void* x, int M, int64_t K, int64_t N, int log2b, const float* absmax,
                     const uint8_t* packed, float* y, const DequantArgs& da, hipStream_t s) {
  return da.K == 16 ? launch_mt<DT, 4>(x, M, K, N, log2b, absmax, packed, y, da, s)
                    : launch_mt<DT, 8>(x, M, K, N, log2b, absmax, packed, y, da, s);
}

}  // namespace

int cu_count() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

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
