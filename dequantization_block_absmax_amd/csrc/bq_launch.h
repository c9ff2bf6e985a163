// bq_launch.h -- kernel launch returning that launch's own status.
//
// hipGetLastError() reports the last error of any earlier HIP call on the thread (a caller's
// event query that returned "not ready", for instance), so launches go through
// hipLaunchKernel, whose return value belongs to this launch alone.  A launch that the
// measurement hook times goes through hipExtLaunchKernel, which stamps the kernel's own start
// and end into two events without putting marker packets between kernels (those left several
// microseconds of idle GPU on each side of the kernel they bracketed).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <tuple>
#include <type_traits>
#include <utility>

#include "bq_internal.h"

namespace bq {

// Compute units of the current device (queried once per device; 256 if the query fails).
int cu_count();

// A launch's threads per dimension (workgroups times workgroup size) must fit in 32 bits;
// larger grids are refused here rather than left to the runtime.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream, Args&&... args) {
  if ((uint64_t)grid.x * block.x > UINT32_MAX || (uint64_t)grid.y * block.y > UINT32_MAX ||
      (uint64_t)grid.z * block.z > UINT32_MAX) {
    g_launch_refused_for_size = true;
    return hipErrorInvalidConfiguration;
  }
  std::tuple<std::decay_t<KArgs>...> vals(std::forward<Args>(args)...);
  return std::apply(
      [&](auto&... v) {
        void* ptrs[] = {static_cast<void*>(&v)...};
        hipEvent_t e0 = static_cast<hipEvent_t>(g_next_launch_start);
        hipEvent_t e1 = static_cast<hipEvent_t>(g_next_launch_stop);
        g_next_launch_start = g_next_launch_stop = nullptr;
        if (e0 != nullptr || e1 != nullptr)
          return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream, e0, e1, 0);
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream);
      },
      vals);
}

}  // namespace bq
