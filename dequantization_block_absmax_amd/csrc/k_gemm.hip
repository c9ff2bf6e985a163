// k_gemm.hip -- fused dequantize + GEMM on the gfx950 matrix cores, for batches of rows
// (gemm_kernel up to 128 rows of x, gemm_tiled_kernel above, gemm_big_kernel for grids of
// 256 x 256 tiles that fill most of the CUs):
// y = x . W16^T, where W16 = RN16(fl32(c[q] * a)) is exactly the 16-bit tensor that
// bq_dequantize_blockwise writes for W, formed in registers and never stored (the
// 16-bit-activation, 4-bit-weight GEMM of "stable-diffusion.cpp PR 2278", Summary, on the
// blockwise codes of this library).
//
//   W: N x K row-major, quantized blockwise over its flat index (element (n, k) is flat
//      element n*K + k); x: M x K row-major, bf16 or fp16 (the type of W16 as well).
//   y[m][n] = sum_k x[m][k] * W16[n][k], products exact in binary32, accumulated in binary32.
//
// Work decomposition.  A workgroup owns an output tile of 32*MT rows of x by 32*NT rows of
// W, and its NW waves split K in chunks of 64 (wave w takes chunks w, w + NW, ...).  Each wave
// computes the whole tile for its chunks with v_mfma_f32_32x32x16 (bf16 or f16): lane l
// (g = l / 32, r = l % 32) supplies A[r][8g + t] and B[8g + t][r], t < 8, and holds
// C[8 (v / 4) + 4 g + v % 4][r] in accumulator element v.  Lane group g takes the 32
// consecutive k from k0 + 32 g of its row: 64 bytes of x (four 16-byte loads) and 16 bytes of
// 4-bit codes (32 of 8-bit), which lie in one block (B >= 32), so one scale serves them.  MFMA
// step s (0..3) uses the lane's k0 + 32 g + 8 s .. + 7 on both operands: the instruction sums
// over 16 values of k, and giving A and B the same assignment of k to lanes and steps leaves
// the product unchanged while every lane feeds the matrix core from its own loads.  The other
// waves' tiles are added to wave 0's through LDS, in wave order, and wave 0 stores y.
#include <hip/hip_runtime.h>

#include "bq_internal.h"
#include "bq_launch.h"

namespace bq {
namespace {

constexpr int kChunk = 64;  // k per wave and chunk (two lane groups of 32)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ f32x16 mfma32x32x16(uint4 a, uint4 b, f32x16 c) {
  if constexpr (DT == BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
}

// Two weights as the 16-bit dequantize stores them: the binary32 products rounded once to the
// 16-bit type (round to nearest even, one packed conversion), first value in the low half.
template <int DT>
__device__ __forceinline__ uint32_t weight_pair(float c0, float c1, float a) {
  f32x2 v = {c0 * a, c1 * a};
  if constexpr (DT == BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  } else {
    // rounded to binary32 first: a fused mixed-precision fma would round the product once
    asm("" : "+v"(v));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
}

// B fragment of MFMA step s: the 8 weights of k offsets 8s .. 8s + 7 of the lane's 32.
//   4-bit: word s of the 16 code bytes; byte b holds offset 2b (high nibble) and 2b + 1.
//   8-bit: words 2s and 2s + 1 of the 32 code bytes, one code per byte.
template <int DT, int KB>
__device__ __forceinline__ uint4 weight_frag(const uint32_t* codes, int s, float a, const float2* s_pair,
                                             const float* s_c) {
  uint32_t w[4];
  if constexpr (KB == 4) {
    const uint32_t word = codes[s];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float2 p = s_pair[(word >> (8 * b)) & 0xffu];
      w[b] = weight_pair<DT>(p.x, p.y, a);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t word = codes[2 * s + h];
      w[2 * h] = weight_pair<DT>(s_c[word & 0xffu], s_c[(word >> 8) & 0xffu], a);
      w[2 * h + 1] = weight_pair<DT>(s_c[(word >> 16) & 0xffu], s_c[word >> 24], a);
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Compiler barrier between a prefetch and the arithmetic on the current chunk (nothing waits
// for the loads here).  The asm memory clobber keeps the prefetch from sinking to its use in
// the next iteration; the scheduling barrier keeps arithmetic on the current chunk, which
// would wait for that chunk's loads, from being scheduled before the prefetch is issued.
__device__ __forceinline__ void prefetch_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// One chunk's operands for a lane: x (MT row tiles x four 16-byte pieces), codes (16 or 32
// bytes per W row tile) and the block scale of each W row tile.
template <int KB, int MT, int NT>
struct Chunk {
  uint4 xa[MT][4];
  uint4 codes[NT][KB == 4 ? 1 : 2];
  float a[NT];
};

template <int DT, int KB, int MT, int NT, int NW>
// x, absmax and packed are not declared __restrict__: the compiler barriers below must order
// their loads, which it may move across a barrier for memory it knows cannot change.
__global__ __launch_bounds__(64 * NW) void gemm_kernel(const uint8_t* x, int64_t M, int64_t K, int64_t N,
                                                        int log2b, const float* absmax, const uint8_t* packed,
                                                        float* __restrict__ y, DequantArgs da) {
  constexpr int kTiles = MT * NT;
  __shared__ float2 s_pair[KB == 4 ? 256 : 1];
  __shared__ float s_c[KB == 8 ? 256 : 1];
  __shared__ float s_red[(NW - 1) * kTiles * 16 * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform in a scalar register: the chunk loop below then branches on scalars, where a
  // loop the compiler takes for divergent joins exec masks and waits for every load there
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r = lane & 31;
  if (tid < 256) {  // 256 table entries (a workgroup has 256 or 512 threads)
    if constexpr (KB == 4) s_pair[tid] = make_float2(da.c[tid >> 4], da.c[tid & 15]);
    else s_c[tid] = da.c[tid];
  }
  __syncthreads();

  const int64_t m0 = (int64_t)blockIdx.y * 32 * MT;
  const int64_t n0 = (int64_t)blockIdx.x * 32 * NT;
  // Rows past M or N read the last row instead (every load is unconditional) and are never
  // stored.
  const uint8_t* xrow[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) xrow[i] = x + (min(m0 + 32 * i + r, M - 1) * K + 32 * g) * 2;
  int64_t wflat[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) wflat[j] = min(n0 + 32 * j + r, N - 1) * K + 32 * g;

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Chunks wave, wave + NW, ...: the loads of a wave's next chunk are issued before its current
  // chunk is dequantized and multiplied (M = 8 at 14336 x 4096: 32.3 us with each chunk's
  // loads waited for in its own iteration).  The chunk index is clamped instead of tested (the
  // last prefetch reads the wave's last chunk again), so no load sits under a condition.
  const int64_t nchunks = K / kChunk;
  const int64_t my_chunks = (nchunks - wave + NW - 1) / NW;  // 0 when wave >= nchunks
  auto load_chunk = [&](int64_t i, Chunk<KB, MT, NT>& c) {
    const int64_t k0 = min((int64_t)wave + (int64_t)NW * i, nchunks - 1) * kChunk;
#pragma unroll
    for (int ii = 0; ii < MT; ++ii)
#pragma unroll
      for (int s = 0; s < 4; ++s) c.xa[ii][s] = *reinterpret_cast<const uint4*>(xrow[ii] + (k0 + 8 * s) * 2);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int64_t f = wflat[j] + k0;
      if constexpr (KB == 4) {
        c.codes[j][0] = *reinterpret_cast<const uint4*>(packed + (f >> 1));
      } else {
        c.codes[j][0] = *reinterpret_cast<const uint4*>(packed + f);
        c.codes[j][1] = *reinterpret_cast<const uint4*>(packed + f + 16);
      }
      c.a[j] = absmax[f >> log2b];
    }
  };
  auto multiply = [&](const Chunk<KB, MT, NT>& c) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 b[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j)
        b[j] = weight_frag<DT, KB>(reinterpret_cast<const uint32_t*>(c.codes[j]), s, c.a[j], s_pair, s_c);
#pragma unroll
      for (int ii = 0; ii < MT; ++ii)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[ii][j] = mfma32x32x16<DT>(c.xa[ii][s], b[j], acc[ii][j]);
    }
  };
  // Two buffers alternate (unrolled by two): copying the prefetched chunk into the current one
  // would make the compiler wait for the prefetch at the end of every iteration.
  // The loop takes two chunks per iteration and has one exit, at the top: a break between its
  // halves would meet the back edge with the break path's prefetch still outstanding, and the
  // compiler would then wait for every load at the top of each iteration.
  Chunk<KB, MT, NT> ca, cb;
  load_chunk(0, ca);
  int64_t i = 0;
  for (; i + 1 < my_chunks; i += 2) {
    load_chunk(i + 1, cb);
    prefetch_fence();
    multiply(ca);
    load_chunk(i + 2, ca);
    prefetch_fence();
    multiply(cb);
  }
  if (i < my_chunks) multiply(ca);  // an odd count: the last chunk, already loaded

  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s_red[(((wave - 1) * kTiles + i * NT + j) * 16 + v) * 64 + lane] = acc[i][j][v];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int64_t col = n0 + 32 * j + r;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float sum = acc[i][j][v];
#pragma unroll
          for (int w = 0; w < NW - 1; ++w) sum += s_red[((w * kTiles + i * NT + j) * 16 + v) * 64 + lane];
          const int64_t row = m0 + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
          if (row < M && col < N) y[row * N + col] = sum;
        }
      }
  }
}

// Large batches: a 128 x 128 output tile per workgroup, its waves arranged 2 x 2 (64 x 64
// each: 2 x 2 accumulator tiles), K in steps of 64 staged through LDS.  Each step, thread t
// loads 32 consecutive k of x row t / 2 and of W row t / 2 (half t % 2), forms the 32 16-bit
// weights, and writes both into the step's LDS buffer; the waves then read standard MFMA
// fragments from LDS, so each x and W16 element is read once per tile.  Two LDS buffers
// alternate (one barrier per step): the next step is formed and written into the other buffer
// between the current step's MFMAs, and a step's global loads are issued two steps ahead.
constexpr int kTileB = 128;        // rows of x and of W per tile
constexpr int kTileK = 64;         // k per step
constexpr int kRowPad = kTileK + 8;  // LDS row stride in 16-bit elements: 144 bytes, so the
                                     // 16-byte fragment reads of 16 lanes hit distinct banks

// (native vectors, not the uint4 struct: a struct copied through LDS stays in scratch memory
// across the compiler barrier)
template <int KB>
struct Stage {
  u32x4 x[4];
  u32x4 codes[KB == 4 ? 1 : 2];
  float a;
};

// One step's global loads for a staging thread: x row and W row (already offset to the
// thread's row and k half), step kt clamped to the last (the last prefetch reads it again).
template <int KB>
__device__ __forceinline__ Stage<KB> load_stage(const uint8_t* xsrc, const uint8_t* packed, const float* absmax,
                                                int64_t wf, int64_t kt, int64_t nk, int log2b) {
  Stage<KB> st;
  const int64_t k0 = min(kt, nk - 1) * kTileK;
#pragma unroll
  for (int s = 0; s < 4; ++s) st.x[s] = *reinterpret_cast<const u32x4*>(xsrc + (k0 + 8 * s) * 2);
  const int64_t f = wf + k0;
  if constexpr (KB == 4) {
    st.codes[0] = *reinterpret_cast<const u32x4*>(packed + (f >> 1));
  } else {
    st.codes[0] = *reinterpret_cast<const u32x4*>(packed + f);
    st.codes[1] = *reinterpret_cast<const u32x4*>(packed + f + 16);
  }
  st.a = absmax[f >> log2b];
  return st;
}

// Writes a staging thread's 32 x values and its 32 16-bit weights into one LDS buffer.
template <int DT, int KB>
__device__ __forceinline__ void store_stage(const Stage<KB>& st, uint16_t* sx, uint16_t* sw, int srow, int shalf,
                                            const float2* s_pair, const float* s_c) {
  uint16_t* xr = sx + srow * kRowPad + 32 * shalf;
  uint16_t* wr = sw + srow * kRowPad + 32 * shalf;
  uint32_t codes[KB == 4 ? 4 : 8];
#pragma unroll
  for (int h = 0; h < (KB == 4 ? 1 : 2); ++h) {
    codes[4 * h] = st.codes[h][0];
    codes[4 * h + 1] = st.codes[h][1];
    codes[4 * h + 2] = st.codes[h][2];
    codes[4 * h + 3] = st.codes[h][3];
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    *reinterpret_cast<u32x4*>(xr + 8 * s) = st.x[s];
    const uint4 w = weight_frag<DT, KB>(codes, s, st.a, s_pair, s_c);
    *reinterpret_cast<u32x4*>(wr + 8 * s) = u32x4{w.x, w.y, w.z, w.w};
  }
}

template <int DT, int KB>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(const uint8_t* x, int64_t M, int64_t K, int64_t N,
                                                         int log2b, const float* absmax, const uint8_t* packed,
                                                         float* __restrict__ y, DequantArgs da) {
  __shared__ float2 s_pair[KB == 4 ? 256 : 1];
  __shared__ float s_c[KB == 8 ? 256 : 1];
  __shared__ __attribute__((aligned(16))) uint16_t s_x[2][kTileB * kRowPad];
  __shared__ __attribute__((aligned(16))) uint16_t s_w[2][kTileB * kRowPad];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  if constexpr (KB == 4) s_pair[tid] = make_float2(da.c[tid >> 4], da.c[tid & 15]);
  else s_c[tid] = da.c[tid];
  __syncthreads();

  const int64_t m0 = (int64_t)blockIdx.y * kTileB;
  const int64_t n0 = (int64_t)blockIdx.x * kTileB;
  // staging: row tid / 2 of both tiles, k half tid % 2; rows past M or N read the last row
  const int srow = tid >> 1, shalf = tid & 1;
  const uint8_t* xsrc = x + (min(m0 + srow, M - 1) * K + 32 * shalf) * 2;
  const int64_t wf = min(n0 + srow, N - 1) * K + 32 * shalf;
  const int64_t nk = K / kTileK;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto multiply = [&](int buf) {
#pragma unroll
    for (int s = 0; s < kTileK / 16; ++s) {
      uint4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const uint4*>(&s_x[buf][(64 * wm + 32 * i + r) * kRowPad + 16 * s + 8 * g]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const uint4*>(&s_w[buf][(64 * wn + 32 * j + r) * kRowPad + 16 * s + 8 * g]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16<DT>(a[i], b[j], acc[i][j]);
    }
  };
  // The step in buffer buf, with the next step (stage st) written into the other buffer piece by
  // piece between its MFMAs, so that the weight formation issues while the MFMAs run.
  auto multiply_store = [&](int buf, const Stage<KB>& st) {
    uint16_t* xr = s_x[buf ^ 1] + srow * kRowPad + 32 * shalf;
    uint16_t* wr = s_w[buf ^ 1] + srow * kRowPad + 32 * shalf;
    uint32_t codes[KB == 4 ? 4 : 8];
#pragma unroll
    for (int h = 0; h < (KB == 4 ? 1 : 2); ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) codes[4 * h + i] = st.codes[h][i];
#pragma unroll
    for (int s = 0; s < kTileK / 16; ++s) {
      uint4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const uint4*>(&s_x[buf][(64 * wm + 32 * i + r) * kRowPad + 16 * s + 8 * g]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const uint4*>(&s_w[buf][(64 * wn + 32 * j + r) * kRowPad + 16 * s + 8 * g]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16<DT>(a[i], b[j], acc[i][j]);
      *reinterpret_cast<u32x4*>(xr + 8 * s) = st.x[s];
      const uint4 w = weight_frag<DT, KB>(codes, s, st.a, s_pair, s_c);
      *reinterpret_cast<u32x4*>(wr + 8 * s) = u32x4{w.x, w.y, w.z, w.w};
    }
  };
  auto load = [&](int64_t kt) { return load_stage<KB>(xsrc, packed, absmax, wf, kt, nk, log2b); };
  // Steps are loaded two ahead, into two register stages that alternate with the two LDS
  // buffers: at the top of each iteration buffer 0 holds step kt and stage s1 step kt + 1
  // (its loads possibly still in flight).  The loop takes two steps and exits only at the top;
  // an odd last step is multiplied after it.
  Stage<KB> s0 = load(0), s1 = load(1);
  store_stage<DT, KB>(s0, s_x[0], s_w[0], srow, shalf, s_pair, s_c);
  __syncthreads();
  int64_t kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    s0 = load(kt + 2);
    prefetch_fence();
    multiply_store(0, s1);  // step kt; step kt + 1 into buffer 1
    __syncthreads();
    s1 = load(kt + 3);
    prefetch_fence();
    multiply_store(1, s0);  // step kt + 1; step kt + 2 into buffer 0
    __syncthreads();
  }
  if (kt < nk) multiply(0);

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + 64 * wn + 32 * j + r;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
        if (row < M && col < N) y[row * N + col] = acc[i][j][v];
      }
    }
}

// Large batches, big tiles: a 256 x TW output tile per workgroup (256 rows of x, TW = 256 or 128
// rows of W), eight waves, each owning 64 columns: arranged 2 x 4 (128 x 64 outputs, 4 x 2
// accumulator tiles) for TW = 256, 4 x 2 (64 x 64, 2 x 2 tiles) for TW = 128; two waves per
// SIMD.  K in LDS-staged steps of 64 with two buffers that alternate.
//
// Staging: the step's tiles are loaded as 16-byte chunks, chunk c of a tile going to thread
// c % 512 (consecutive threads take consecutive chunks of a row, so each load instruction
// covers whole rows): x has 8 chunks per row (64 k), W 2 (4-bit codes, 32 k each) or 4 (8-bit,
// 16 k each), each W chunk with the scale of its block (B >= 32, so one scale serves a chunk).
// With 128 rows of 4-bit codes (256 chunks) the first four waves stage W.
// A step's loads are issued one step ahead into one of two register stages, and the stage of
// the next step is formed and written into the other LDS buffer a quarter at a time between
// the current step's MFMAs.
constexpr int kBigM = 256;
constexpr int kBigThreads = 512;

template <int KB, int TW>
struct BigStage {
  static constexpr int kWtot = TW * (KB == 4 ? 2 : 4);  // W chunks per tile
  static constexpr int kW = kWtot >= kBigThreads ? kWtot / kBigThreads : 1;  // per thread
  u32x4 x[4];
  u32x4 w[kW];
  float a[kW];
};

template <int DT, int KB, int TW>
__global__ __launch_bounds__(kBigThreads, 1) void gemm_big_kernel(const uint8_t* x, int64_t M, int64_t K,
                                                                  int64_t N, int log2b, const float* absmax,
                                                                  const uint8_t* packed, float* __restrict__ y,
                                                                  DequantArgs da) {
  constexpr int WGN = TW / 64;            // waves along W (64 columns each)
  constexpr int NI = 256 / (8 / WGN) / 32, NJ = 2;  // accumulator tiles per wave
  constexpr int kCpr = KB == 4 ? 2 : 4;   // W chunks per row
  constexpr int kW = BigStage<KB, TW>::kW;
  const bool wstage = BigStage<KB, TW>::kWtot >= kBigThreads || threadIdx.x < BigStage<KB, TW>::kWtot;  // uniform per wave
  __shared__ float2 s_pair[KB == 4 ? 256 : 1];
  __shared__ float s_c[KB == 8 ? 256 : 1];
  __shared__ __attribute__((aligned(16))) uint16_t s_x[2][kBigM * kRowPad];
  __shared__ __attribute__((aligned(16))) uint16_t s_w[2][TW * kRowPad];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r = lane & 31;
  const int wm = wave / WGN, wn = wave % WGN;
  if (tid < 256) {
    if constexpr (KB == 4) s_pair[tid] = make_float2(da.c[tid >> 4], da.c[tid & 15]);
    else s_c[tid] = da.c[tid];
  }
  __syncthreads();

  const int64_t m0 = (int64_t)blockIdx.y * kBigM;
  const int64_t n0 = (int64_t)blockIdx.x * TW;
  const int64_t nk = K / kTileK;
  // x chunk i of this thread: row 64 i + tid / 8 of the tile, bytes 16 (tid % 8) of its 128;
  // rows past M read the last row and are never stored
  const uint8_t* xsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xsrc[i] = x + (min(m0 + 64 * i + (tid >> 3), M - 1) * K) * 2 + 16 * (tid & 7);
  // W chunk i of this thread: c = 512 i + tid, row c / kCpr, chunk c % kCpr
  int64_t wflat[kW];
#pragma unroll
  for (int i = 0; i < kW; ++i) {
    const int c = kBigThreads * i + tid;
    wflat[i] = min(n0 + c / kCpr, N - 1) * K + (c % kCpr) * (KB == 4 ? 32 : 16);
  }

  f32x16 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto load = [&](int64_t kt, BigStage<KB, TW>& st) {
    const int64_t k0 = min(kt, nk - 1) * kTileK;
#pragma unroll
    for (int i = 0; i < 4; ++i) st.x[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + k0 * 2);
#pragma unroll
    for (int i = 0; i < kW; ++i) {
      if (!wstage) break;
      const int64_t f = wflat[i] + k0;
      st.w[i] = *reinterpret_cast<const u32x4*>(packed + (KB == 4 ? (f >> 1) : f));
      st.a[i] = absmax[f >> log2b];
    }
  };
  // Quarter q of a stage into LDS buffer buf: x chunk q, and a quarter of each W chunk's
  // weights (4-bit: 8 of its 32; 8-bit: 4 of its 16).
  auto store_quarter = [&](const BigStage<KB, TW>& st, int buf, int q) {
    *reinterpret_cast<u32x4*>(&s_x[buf][(64 * q + (tid >> 3)) * kRowPad + 8 * (tid & 7)]) = st.x[q];
#pragma unroll
    for (int i = 0; i < kW; ++i) {
      if (!wstage) break;
      const int c = kBigThreads * i + tid;
      const int row = c / kCpr, ch = c % kCpr;
      const uint32_t word = st.w[i][q];
      if constexpr (KB == 4) {
        u32x4 w;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float2 pr = s_pair[(word >> (8 * b)) & 0xffu];
          w[b] = weight_pair<DT>(pr.x, pr.y, st.a[i]);
        }
        *reinterpret_cast<u32x4*>(&s_w[buf][row * kRowPad + 32 * ch + 8 * q]) = w;
      } else {
        uint2 w;
        w.x = weight_pair<DT>(s_c[word & 0xffu], s_c[(word >> 8) & 0xffu], st.a[i]);
        w.y = weight_pair<DT>(s_c[(word >> 16) & 0xffu], s_c[word >> 24], st.a[i]);
        *reinterpret_cast<uint2*>(&s_w[buf][row * kRowPad + 16 * ch + 4 * q]) = w;
      }
    }
  };
  auto frags = [&](int buf, int s, uint4 (&fa)[NI], uint4 (&fb)[NJ]) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      fa[i] = *reinterpret_cast<const uint4*>(&s_x[buf][(32 * NI * wm + 32 * i + r) * kRowPad + 16 * s + 8 * g]);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      fb[j] = *reinterpret_cast<const uint4*>(&s_w[buf][(64 * wn + 32 * j + r) * kRowPad + 16 * s + 8 * g]);
  };
  // The step in buffer buf; with st, the next step's stage is written into the other buffer
  // a quarter per 16-k piece.  The fragments of piece s + 1 are read before the MFMAs of piece s.
  auto multiply = [&](int buf, const BigStage<KB, TW>* st) {
    uint4 fa[2][NI], fb[2][NJ];
    frags(buf, 0, fa[0], fb[0]);
#pragma unroll
    for (int s = 0; s < kTileK / 16; ++s) {
      if (s + 1 < kTileK / 16) frags(buf, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32x32x16<DT>(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
      if (st != nullptr) store_quarter(*st, buf ^ 1, s);
    }
  };

  BigStage<KB, TW> s0, s1;
  load(0, s0);
  load(1, s1);
#pragma unroll
  for (int q = 0; q < 4; ++q) store_quarter(s0, 0, q);
  __syncthreads();
  int64_t kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    load(kt + 2, s0);
    prefetch_fence();
    multiply(0, &s1);  // step kt; step kt + 1 into buffer 1
    __syncthreads();
    load(kt + 3, s1);
    prefetch_fence();
    multiply(1, &s0);  // step kt + 1; step kt + 2 into buffer 0
    __syncthreads();
  }
  if (kt < nk) multiply(0, nullptr);

#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t col = n0 + 64 * wn + 32 * j + r;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + 32 * NI * wm + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
        if (row < M && col < N) y[row * N + col] = acc[i][j][v];
      }
    }
}

// 64 rows of W per workgroup (two column tiles: x is loaded once for both), 32, 64 or 128 rows
// of x, and NW waves splitting K.  Measured at 14336 x 4096 against 32 rows of W and against
// other wave counts: 8 waves for 32 rows of x (M = 8: 17.4 against 21.7 us with 4; the grid
// has only N / 64 workgroups, so more waves hide more latency), 4 waves for more rows (M = 64:
// 30.6 against 34.0 us with 8).  128-row tiles from M = 65 share each dequantized weight
// among more rows (M = 128: 49.1 against 52.6 us with 64-row tiles).
template <int DT, int KB, int MT, int NW>
hipError_t launch_mt(const void* x, int64_t M, int64_t K, int64_t N, int log2b, const float* absmax,
                     const uint8_t* packed, float* y, const DequantArgs& da, hipStream_t s) {
  constexpr int NT = 2;
  const dim3 grid((unsigned)((N + 32 * NT - 1) / (32 * NT)), (unsigned)((M + 32 * MT - 1) / (32 * MT)));
  return launch_kernel(gemm_kernel<DT, KB, MT, NT, NW>, grid, dim3(64 * NW), s, static_cast<const uint8_t*>(x), M,
                       K, N, log2b, absmax, packed, y, da);
}

template <int DT, int KB>
hipError_t launch_kb(const void* x, int64_t M, int64_t K, int64_t N, int log2b, const float* absmax,
                     const uint8_t* packed, float* y, const DequantArgs& da, hipStream_t s) {
  if (M <= 32) return launch_mt<DT, KB, 1, 8>(x, M, K, N, log2b, absmax, packed, y, da, s);
  if (M <= 64) return launch_mt<DT, KB, 2, 4>(x, M, K, N, log2b, absmax, packed, y, da, s);
  // Above 128 rows the LDS-tiled kernels: x and W16 read once per tile (at 14336 x 4096: M =
  // 256 56.4 against 95.3 us with the register-tiled kernel, M = 1024 181 against 335; M = 128
  // 55.6 against 52.1).
  if (M <= 128) return launch_mt<DT, KB, 4, 4>(x, M, K, N, log2b, absmax, packed, y, da, s);
  // 256-row tiles (one workgroup fills a CU).  256 x 128 tiles when they fill at least three
  // quarters of the CUs in one round: at 14336 x 4096, M = 512 (224 tiles) 4-bit 77 against
  // 90 us in the 128 x 128 form, 8-bit 84 against 108; M = 384 75 against 82 and 80 against
  // 102.  Otherwise 256 x 256 tiles when they fill at least half of the CUs: M = 1024 (224
  // tiles), 4-bit 131-144 against 176-184 us in the 128 x 128 form, 8-bit 143-160 against
  // 180-195 in a 256 x 128 form that loads x straight into fragments; M = 2048 269 against
  // 332 (4-bit); M = 768 (168 tiles) about the M = 1024 time, against 138 (in two rounds of
  // 256 x 128 tiles 146).  Smaller grids keep the 128 x 128 form, two workgroups per CU.
  const int64_t mt = (M + kBigM - 1) / kBigM;
  const int64_t cus = cu_count();
  const int64_t t128 = ((N + 127) / 128) * mt, t256 = ((N + 255) / 256) * mt;
  if (t128 <= cus && 4 * t128 >= 3 * cus) {
    const dim3 grid((unsigned)((N + 127) / 128), (unsigned)mt);
    return launch_kernel(gemm_big_kernel<DT, KB, 128>, grid, dim3(kBigThreads), s, static_cast<const uint8_t*>(x), M,
                         K, N, log2b, absmax, packed, y, da);
  }
  if (2 * t256 >= cus) {
    const dim3 grid((unsigned)((N + 255) / 256), (unsigned)mt);
    return launch_kernel(gemm_big_kernel<DT, KB, 256>, grid, dim3(kBigThreads), s, static_cast<const uint8_t*>(x), M,
                         K, N, log2b, absmax, packed, y, da);
  }
  const dim3 grid((unsigned)((N + kTileB - 1) / kTileB), (unsigned)((M + kTileB - 1) / kTileB));
  return launch_kernel(gemm_tiled_kernel<DT, KB>, grid, dim3(256), s, static_cast<const uint8_t*>(x), M, K, N,
                       log2b, absmax, packed, y, da);
}

}  // namespace

int launch_gemm(const void* x, int dtype, int64_t M, int64_t K, int64_t N, int blocksize, const DequantArgs& da,
                const float* absmax, const uint8_t* packed, float* y, void* stream) {
  int log2b = 0;
  while ((1 << log2b) < blocksize) ++log2b;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == BF16)
    e = da.K == 16 ? launch_kb<BF16, 4>(x, M, K, N, log2b, absmax, packed, y, da, s)
                   : launch_kb<BF16, 8>(x, M, K, N, log2b, absmax, packed, y, da, s);
  else
    e = da.K == 16 ? launch_kb<F16, 4>(x, M, K, N, log2b, absmax, packed, y, da, s)
                   : launch_kb<F16, 8>(x, M, K, N, log2b, absmax, packed, y, da, s);
  return (int)e;
}

}  // namespace bq
