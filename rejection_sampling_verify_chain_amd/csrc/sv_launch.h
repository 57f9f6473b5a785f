// Kernel launch helper: hipLaunchKernel with per-argument conversion to the kernel's parameter
// types, returning the launch status directly, and optional per-kernel event timing.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

namespace sv {

// Kernel timing (see sv_trace_* in the C ABI).  When tracing is on, trace_slot hands out the
// next pair of events and the kernel is launched with hipExtLaunchKernel, which stamps them
// with the start and end time of the kernel's own execution (no gap before or after it).
bool trace_on();
bool trace_slot(const char* name, hipEvent_t* begin, hipEvent_t* end);

template <typename... KArgs, typename... Args>
hipError_t launch_kernel_shm(const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                             size_t shared_bytes, hipStream_t stream, Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count mismatch");
  std::tuple<KArgs...> held(static_cast<KArgs>(std::forward<Args>(args))...);
  void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply(
      [&](auto&... e) {
        int i = 0;
        ((ptrs[i++] = static_cast<void*>(&e)), ...);
      },
      held);
  hipEvent_t t0 = nullptr, t1 = nullptr;
  if (trace_on() && trace_slot(name, &t0, &t1))
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs,
                              shared_bytes, stream, t0, t1, 0);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shared_bytes,
                         stream);
}

template <typename... KArgs, typename... Args>
hipError_t launch_kernel(const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                         hipStream_t stream, Args&&... args) {
  return launch_kernel_shm(name, kernel, grid, block, 0, stream, std::forward<Args>(args)...);
}

}  // namespace sv
