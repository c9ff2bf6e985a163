// k_scratch.hip -- the library's own scratch memory, for bq_quantize_nested_noalloc.
//
// A nested quantize needs a workspace for the block maxima and the per-wave partial sums of the
// mean.  Callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc) use this fixed array instead of one of their
// own.  It is a file-scope device variable: each GPU the library runs on holds its own copy,
// allocated when the code object is loaded and kept until the process ends.  In host code the
// array's name is only a host-side stand-in, so its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and kept; kernels receive that
// address, never the name.  Every call on one GPU shares the array: calls that overlap on one
// GPU (two streams, or two host threads) race on it.  Nothing in it has to start at zero: the
// data pass writes every word the statistics kernels read.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bq_internal.h"

namespace bq {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int scratch_buffer(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

}  // namespace bq
