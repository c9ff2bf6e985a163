// bq_launch.h -- kernel launch returning that launch's own status.
//
// hipGetLastError() reports the last error of any earlier HIP call on the thread (a caller's
// event query that returned "not ready", for instance), so launches go through
// hipLaunchKernel, whose return value belongs to this launch alone.
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>
#include <type_traits>
#include <utility>

namespace bq {

template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream, Args&&... args) {
  std::tuple<std::decay_t<KArgs>...> vals(std::forward<Args>(args)...);
  return std::apply(
      [&](auto&... v) {
        void* ptrs[] = {static_cast<void*>(&v)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream);
      },
      vals);
}

}  // namespace bq
