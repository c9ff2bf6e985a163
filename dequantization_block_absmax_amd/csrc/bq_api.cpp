// bq_api.cpp -- the C ABI of libbq (declared in include/bq.h).
//
// Each entry point validates everything on the host first (validation once, at the
// interface: the boundary checks of "[OMNIML-5899] Add CUDA kernels for IQ packing"), then
// enqueues its kernels on the caller's stream ("Respect the current CUDA stream in blockwise
// quantization", bitsandbytes PR 2052).  Tables are passed to kernels by value: no
// allocation, no host-to-device copy and no synchronization per call (the per-call constant
// upload measured in "Cache device-side constants in dequant kernels", ComfyUI-GGUF PR 472,
// "Problem", and the graph-capture limitation in PR 2052, "Limitations").
#include <hip/hip_runtime_api.h>
#include <string.h>

#include <mutex>

#include "bq.h"
#include "bq_debug.h"
#include "bq_internal.h"

namespace {

bool valid_dtype(bq_dtype d) { return d == BQ_F32 || d == BQ_F16 || d == BQ_BF16; }

bool valid_blocksize(int32_t b) {
  for (int v = 32; v <= 4096; v *= 2)
    if (b == v) return true;
  return false;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

thread_local int g_last_hip_error = 0;

bq_status hip_status(int e) {
  const bool refused = bq::g_launch_refused_for_size;
  bq::g_launch_refused_for_size = false;
  if (e == 0) return BQ_OK;
  // the launcher's own refusal of a grid over 2^32 - 1 threads (no launch was made); the same
  // error code from the runtime is a failed launch like any other
  if (refused && e == (int)hipErrorInvalidConfiguration) return BQ_ERR_SIZE;
  g_last_hip_error = e;
  return BQ_ERR_HIP;
}

int64_t nblocks(int64_t n, int32_t b) { return (n + b - 1) / b; }

// Nested workspace: the block maxima (binary32 absmax[nb] for fp32 input, the 16-bit patterns
// for fp16 / bf16 input, in the same region), padded to 256 bytes, then one binary64 run sum
// of the mean's tree per kRunBlocks blocks.
size_t ws_runs_offset(int64_t nb) { return ((size_t)nb * 4 + 255) & ~(size_t)255; }

size_t ws_bytes(int64_t nb) {
  return ws_runs_offset(nb) + (size_t)((nb + bq::kRunBlocks - 1) / bq::kRunBlocks) * 8;
}

// Preparing a table (validation, thresholds, bucket LUT) costs more host time than a small
// launch, so the last few prepared tables are kept, keyed by their entries.  This is a
// host-side memo only: results never depend on it.
struct TableCache {
  static constexpr int kSlots = 8;
  struct Slot {
    int size = 0;
    float entries[256];
    bq::PreparedTable table;
  };
  std::mutex mu;
  Slot slots[kSlots];
  int next = 0;

  bool lookup(const float* e, int size, bq::PreparedTable* out) {
    std::lock_guard<std::mutex> g(mu);
    for (Slot& s : slots)
      if (s.size == size && memcmp(s.entries, e, sizeof(float) * size) == 0) {
        memcpy(out, &s.table, sizeof(*out));
        return true;
      }
    return false;
  }
  void insert(const float* e, int size, const bq::PreparedTable& t) {
    std::lock_guard<std::mutex> g(mu);
    Slot& s = slots[next];
    next = (next + 1) % kSlots;
    s.size = size;
    memcpy(s.entries, e, sizeof(float) * size);
    memcpy(&s.table, &t, sizeof(t));
  }
};

TableCache& table_cache() {
  static TableCache* c = new TableCache();  // never destroyed: usable during process exit
  return *c;
}

bq_status check_table(const bq_code_table* t, bq::PreparedTable* out) {
  if (t == nullptr || t->entries == nullptr) return BQ_ERR_NULL;
  if (t->size != 16 && t->size != 256) return BQ_ERR_TABLE;
  if (table_cache().lookup(t->entries, t->size, out)) return BQ_OK;
  if (!bq::prepare_table(t->entries, t->size, out)) return BQ_ERR_TABLE;
  table_cache().insert(t->entries, t->size, *out);
  return BQ_OK;
}

// Scratch for prepared tables: prepared per call on the host, never shared between calls.
struct Tables {
  bq::PreparedTable data, stats;
};

}  // namespace

extern "C" {

int bq_last_hip_error(void) { return g_last_hip_error; }

bq_status bq_debug_time_next_kernel(hipEvent_t start, hipEvent_t stop) {
  bq::g_next_launch_start = start;
  bq::g_next_launch_stop = stop;
  return BQ_OK;
}

const char* bq_status_string(bq_status s) {
  switch (s) {
    case BQ_OK: return "ok";
    case BQ_ERR_NULL: return "a required pointer is NULL";
    case BQ_ERR_DTYPE: return "unknown dtype";
    case BQ_ERR_SIZE: return "invalid element count";
    case BQ_ERR_BLOCKSIZE: return "block size must be a power of two in [32, 4096]";
    case BQ_ERR_TABLE: return "invalid code table";
    case BQ_ERR_ALIGNMENT: return "misaligned device pointer";
    case BQ_ERR_FORMAT: return "unknown block format or row length";
    case BQ_ERR_WORKSPACE: return "nested workspace missing or too small";
    case BQ_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

bq_status bq_quantize_blockwise(const void* in, bq_dtype dtype, int64_t n, int32_t blocksize,
                                const bq_code_table* code_table, float* absmax, uint8_t* packed,
                                hipStream_t stream) {
  if (!valid_dtype(dtype)) return BQ_ERR_DTYPE;
  if (n < 0) return BQ_ERR_SIZE;
  if (!valid_blocksize(blocksize)) return BQ_ERR_BLOCKSIZE;
  Tables t;
  bq_status st = check_table(code_table, &t.data);
  if (st != BQ_OK) return st;
  if (n == 0) return BQ_OK;
  if (in == nullptr || absmax == nullptr || packed == nullptr) return BQ_ERR_NULL;
  if (nblocks(n, blocksize) > INT32_MAX) return BQ_ERR_SIZE;
  if (!aligned(in, 16) || !aligned(packed, 16) || !aligned(absmax, 4)) return BQ_ERR_ALIGNMENT;
  return hip_status(bq::launch_quantize(in, dtype, n, blocksize, t.data, absmax, packed, false, stream));
}

bq_status bq_dequantize_blockwise(void* out, bq_dtype dtype, int64_t n, int32_t blocksize,
                                  const bq_code_table* code_table, const float* absmax,
                                  const uint8_t* packed, hipStream_t stream) {
  if (!valid_dtype(dtype)) return BQ_ERR_DTYPE;
  if (n < 0) return BQ_ERR_SIZE;
  if (!valid_blocksize(blocksize)) return BQ_ERR_BLOCKSIZE;
  Tables t;
  bq_status st = check_table(code_table, &t.data);
  if (st != BQ_OK) return st;
  if (n == 0) return BQ_OK;
  if (out == nullptr || absmax == nullptr || packed == nullptr) return BQ_ERR_NULL;
  if (nblocks(n, blocksize) > INT32_MAX) return BQ_ERR_SIZE;
  if (!aligned(out, 16) || !aligned(packed, 16) || !aligned(absmax, 4)) return BQ_ERR_ALIGNMENT;
  bq::DequantArgs a;
  memset(&a, 0, sizeof(a));
  memcpy(a.c, t.data.c, sizeof(float) * t.data.K);
  a.K = t.data.K;
  return hip_status(bq::launch_dequantize(out, dtype, n, blocksize, a, absmax, packed, stream));
}

bq_status bq_linear_blockwise(const void* x, bq_dtype dtype, int64_t M, int64_t K, int64_t N, int32_t blocksize,
                              const bq_code_table* code_table, const float* absmax, const uint8_t* packed,
                              float* y, hipStream_t stream) {
  if (!valid_dtype(dtype)) return BQ_ERR_DTYPE;
  if (M < 1 || M > 4 || K <= 0 || K % 16 != 0 || N < 0) return BQ_ERR_SIZE;
  if (N > 0 && K > INT64_MAX / N) return BQ_ERR_SIZE;
  if (!valid_blocksize(blocksize)) return BQ_ERR_BLOCKSIZE;
  Tables t;
  bq_status st = check_table(code_table, &t.data);
  if (st != BQ_OK) return st;
  if (N == 0) return BQ_OK;
  if (x == nullptr || absmax == nullptr || packed == nullptr || y == nullptr) return BQ_ERR_NULL;
  // at least 4 rows per workgroup of 256 threads, and a launch holds at most 2^32 - 1 threads
  if (nblocks(N * K, blocksize) > INT32_MAX || (N + 3) / 4 * 256 > UINT32_MAX) return BQ_ERR_SIZE;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(absmax, 4) || !aligned(y, 4)) return BQ_ERR_ALIGNMENT;
  bq::DequantArgs a;
  memset(&a, 0, sizeof(a));
  memcpy(a.c, t.data.c, sizeof(float) * t.data.K);
  a.K = t.data.K;
  return hip_status(bq::launch_linear(x, dtype, M, K, N, blocksize, a, absmax, packed, y, stream));
}

bq_status bq_gemm_blockwise(const void* x, bq_dtype dtype, int64_t M, int64_t K, int64_t N, int32_t blocksize,
                            const bq_code_table* code_table, const float* absmax, const uint8_t* packed,
                            float* y, hipStream_t stream) {
  if (dtype != BQ_BF16 && dtype != BQ_F16) return BQ_ERR_DTYPE;
  // grid rows: ceil(M / 64) <= 65535
  if (M < 1 || M > 65535 * 64 || K <= 0 || K % 64 != 0 || N < 0) return BQ_ERR_SIZE;
  if (N > 0 && K > INT64_MAX / N) return BQ_ERR_SIZE;
  if (M > INT64_MAX / K || (N > 0 && M > INT64_MAX / N)) return BQ_ERR_SIZE;
  if (!valid_blocksize(blocksize)) return BQ_ERR_BLOCKSIZE;
  Tables t;
  bq_status st = check_table(code_table, &t.data);
  if (st != BQ_OK) return st;
  if (N == 0) return BQ_OK;
  if (x == nullptr || absmax == nullptr || packed == nullptr || y == nullptr) return BQ_ERR_NULL;
  // at least 64 columns per workgroup of at most 512 threads; at most 2^32 - 1 threads a launch
  if (nblocks(N * K, blocksize) > INT32_MAX || (N + 63) / 64 * 512 > UINT32_MAX) return BQ_ERR_SIZE;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(absmax, 4) || !aligned(y, 4)) return BQ_ERR_ALIGNMENT;
  bq::DequantArgs a;
  memset(&a, 0, sizeof(a));
  memcpy(a.c, t.data.c, sizeof(float) * t.data.K);
  a.K = t.data.K;
  return hip_status(bq::launch_gemm(x, dtype, M, K, N, blocksize, a, absmax, packed, y, stream));
}

size_t bq_nested_workspace_bytes(int64_t n, int32_t blocksize, int32_t blocksize2) {
  (void)blocksize2;
  if (n <= 0 || !valid_blocksize(blocksize)) return 0;
  return ws_bytes(nblocks(n, blocksize));
}

static bq_status check_nested(const bq_nested_stats* stats, bq::PreparedTable* t2, bool need_ws,
                              int64_t n, int32_t blocksize) {
  if (stats == nullptr) return BQ_ERR_NULL;
  if (!valid_blocksize(stats->blocksize2)) return BQ_ERR_BLOCKSIZE;
  bq_status st = check_table(stats->table, t2);
  if (st != BQ_OK) return st;
  if (t2->K != 256) return BQ_ERR_TABLE;
  if (n == 0) return BQ_OK;
  if (stats->qabsmax == nullptr || stats->absmax2 == nullptr || stats->mean == nullptr) return BQ_ERR_NULL;
  if (!aligned(stats->qabsmax, 16) || !aligned(stats->absmax2, 4) || !aligned(stats->mean, 4)) return BQ_ERR_ALIGNMENT;
  if (need_ws) {
    if (stats->workspace == nullptr) return BQ_ERR_WORKSPACE;
    if (!aligned(stats->workspace, 256)) return BQ_ERR_ALIGNMENT;
    if (stats->workspace_bytes < ws_bytes(nblocks(n, blocksize))) return BQ_ERR_WORKSPACE;
  }
  return BQ_OK;
}

// Validation of a nested quantize; the workspace is checked only when the caller brings it.
static bq_status check_quantize_nested(const void* in, bq_dtype dtype, int64_t n, int32_t blocksize,
                                       const bq_code_table* code_table, const bq_nested_stats* stats,
                                       const uint8_t* packed, bool caller_ws, Tables* t) {
  if (!valid_dtype(dtype)) return BQ_ERR_DTYPE;
  if (n < 0) return BQ_ERR_SIZE;
  if (!valid_blocksize(blocksize)) return BQ_ERR_BLOCKSIZE;
  bq_status st = check_table(code_table, &t->data);
  if (st != BQ_OK) return st;
  st = check_nested(stats, &t->stats, caller_ws, n, blocksize);
  if (st != BQ_OK) return st;
  if (n == 0) return BQ_OK;
  if (in == nullptr || packed == nullptr) return BQ_ERR_NULL;
  if (nblocks(n, blocksize) > INT32_MAX) return BQ_ERR_SIZE;
  if (!aligned(in, 16) || !aligned(packed, 16)) return BQ_ERR_ALIGNMENT;
  return BQ_OK;
}

// The launches of a validated nested quantize (n > 0) with workspace `ws`.
static bq_status launch_quantize_nested(const void* in, bq_dtype dtype, int64_t n, int32_t blocksize,
                                        const Tables& t, const bq_nested_stats* stats, uint8_t* packed, void* ws,
                                        hipStream_t stream) {
  const int64_t nb = nblocks(n, blocksize);
  void* ws_absmax = ws;
  double* ws_runs = reinterpret_cast<double*>(static_cast<uint8_t*>(ws) + ws_runs_offset(nb));
  int e = bq::launch_quantize(in, dtype, n, blocksize, t.data, ws_absmax, packed, true, stream);
  if (e != 0) return hip_status(e);
  e = bq::launch_nested_stats(ws_absmax, dtype, nb, stats->blocksize2, t.stats, ws_runs, stats->qabsmax,
                              stats->absmax2, stats->mean, stream);
  return hip_status(e);
}

bq_status bq_quantize_nested(const void* in, bq_dtype dtype, int64_t n, int32_t blocksize,
                             const bq_code_table* code_table, bq_nested_stats* stats,
                             uint8_t* packed, hipStream_t stream) {
  Tables t;
  const bq_status st = check_quantize_nested(in, dtype, n, blocksize, code_table, stats, packed, true, &t);
  if (st != BQ_OK || n == 0) return st;
  return launch_quantize_nested(in, dtype, n, blocksize, t, stats, packed, stats->workspace, stream);
}

bq_status bq_quantize_nested_noalloc(const void* in, bq_dtype dtype, int64_t n, int32_t blocksize,
                                     const bq_code_table* code_table, bq_nested_stats* stats,
                                     uint8_t* packed, hipStream_t stream) {
  Tables t;
  const bq_status st = check_quantize_nested(in, dtype, n, blocksize, code_table, stats, packed, false, &t);
  if (st != BQ_OK || n == 0) return st;
  if (ws_bytes(nblocks(n, blocksize)) > bq::kScratchBytes) return BQ_ERR_WORKSPACE;
  void* scratch = nullptr;
  const int e = bq::scratch_buffer(&scratch);
  if (e != 0) return hip_status(e);
  return launch_quantize_nested(in, dtype, n, blocksize, t, stats, packed, scratch, stream);
}

bq_status bq_dequantize_nested(void* out, bq_dtype dtype, int64_t n, int32_t blocksize,
                               const bq_code_table* code_table, const bq_nested_stats* stats,
                               const uint8_t* packed, hipStream_t stream) {
  if (!valid_dtype(dtype)) return BQ_ERR_DTYPE;
  if (n < 0) return BQ_ERR_SIZE;
  if (!valid_blocksize(blocksize)) return BQ_ERR_BLOCKSIZE;
  Tables t;
  bq_status st = check_table(code_table, &t.data);
  if (st != BQ_OK) return st;
  st = check_nested(stats, &t.stats, false, n, blocksize);
  if (st != BQ_OK) return st;
  if (n == 0) return BQ_OK;
  if (out == nullptr || packed == nullptr) return BQ_ERR_NULL;
  if (nblocks(n, blocksize) > INT32_MAX) return BQ_ERR_SIZE;
  if (!aligned(out, 16) || !aligned(packed, 16)) return BQ_ERR_ALIGNMENT;
  bq::NestedDequantArgs a;
  memset(&a, 0, sizeof(a));
  memcpy(a.c, t.data.c, sizeof(float) * t.data.K);
  memcpy(a.c2, t.stats.c, sizeof(float) * 256);
  a.K = t.data.K;
  return hip_status(bq::launch_dequantize_nested(out, dtype, n, blocksize, stats->blocksize2, a, stats->qabsmax,
                                                 stats->absmax2, stats->mean, packed, stream));
}

bq_status bq_dequant_q32(const void* blocks, bq_dtype dtype, int64_t n, int32_t row_len,
                         bq_q32_format format, void* out, hipStream_t stream) {
  if (!valid_dtype(dtype)) return BQ_ERR_DTYPE;
  if (format != BQ_Q32_Q4 && format != BQ_Q32_Q8) return BQ_ERR_FORMAT;
  if (row_len <= 0 || row_len % 32 != 0) return BQ_ERR_FORMAT;
  if (n < 0 || n % row_len != 0) return BQ_ERR_SIZE;
  if (n == 0) return BQ_OK;
  if (blocks == nullptr || out == nullptr) return BQ_ERR_NULL;
  if (n / 32 > INT32_MAX) return BQ_ERR_SIZE;
  if (!aligned(blocks, 2) || !aligned(out, 16)) return BQ_ERR_ALIGNMENT;
  return hip_status(bq::launch_q32(blocks, dtype, n, (int)format, out, stream));
}

static bq_status check_superblock_shape(bq_dtype dtype, int64_t n, int64_t row_len) {
  if (!valid_dtype(dtype)) return BQ_ERR_DTYPE;
  if (row_len <= 0 || row_len % 256 != 0) return BQ_ERR_FORMAT;
  if (n < 0 || n % row_len != 0 || n / 256 > INT32_MAX) return BQ_ERR_SIZE;
  return BQ_OK;
}

bq_status bq_iq2xs_quantize(const void* in, bq_dtype dtype, int64_t n, int64_t row_len, const uint8_t* grid,
                            const uint16_t* scales, uint8_t* blocks, uint32_t* rejected, hipStream_t stream) {
  const bq_status st = check_superblock_shape(dtype, n, row_len);
  if (st != BQ_OK || n == 0) return st;
  if (in == nullptr || grid == nullptr || scales == nullptr || blocks == nullptr || rejected == nullptr)
    return BQ_ERR_NULL;
  if (!aligned(in, 16) || !aligned(grid, 16) || !aligned(scales, 2) || !aligned(blocks, 2) || !aligned(rejected, 4))
    return BQ_ERR_ALIGNMENT;
  return hip_status(bq::launch_iq2xs_quantize(in, dtype, n, grid, scales, blocks, rejected, stream));
}

bq_status bq_iq1s_quantize(const void* in, bq_dtype dtype, int64_t n, int64_t row_len, const int8_t* grid,
                           uint8_t* blocks, hipStream_t stream) {
  const bq_status st = check_superblock_shape(dtype, n, row_len);
  if (st != BQ_OK || n == 0) return st;
  if (in == nullptr || grid == nullptr || blocks == nullptr) return BQ_ERR_NULL;
  if (!aligned(in, 16) || !aligned(grid, 16) || !aligned(blocks, 2)) return BQ_ERR_ALIGNMENT;
  return hip_status(bq::launch_iq1s_quantize(in, dtype, n, grid, blocks, stream));
}

bq_status bq_iq1s_dequantize(const uint8_t* blocks, const int8_t* grid, int64_t n, int64_t row_len,
                             bq_dtype dtype, void* out, hipStream_t stream) {
  const bq_status st = check_superblock_shape(dtype, n, row_len);
  if (st != BQ_OK || n == 0) return st;
  if (blocks == nullptr || grid == nullptr || out == nullptr) return BQ_ERR_NULL;
  if (!aligned(blocks, 2) || !aligned(grid, 8) || !aligned(out, 16)) return BQ_ERR_ALIGNMENT;
  return hip_status(bq::launch_iq1s_dequantize(blocks, grid, n, dtype, out, stream));
}

bq_status bq_iq2xs_dequantize(const uint8_t* blocks, const uint8_t* grid, int64_t n, int64_t row_len,
                              bq_dtype dtype, void* out, hipStream_t stream) {
  const bq_status st = check_superblock_shape(dtype, n, row_len);
  if (st != BQ_OK || n == 0) return st;
  if (blocks == nullptr || grid == nullptr || out == nullptr) return BQ_ERR_NULL;
  if (!aligned(blocks, 2) || !aligned(grid, 8) || !aligned(out, 16)) return BQ_ERR_ALIGNMENT;
  return hip_status(bq::launch_iq2xs_dequantize(blocks, grid, n, dtype, out, stream));
}

}  // extern "C"
