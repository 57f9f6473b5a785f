// Kernel launch helper: hipLaunchKernel with per-argument conversion to the kernel's parameter
// types, returning the launch status directly, and optional per-kernel event timing.
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

namespace sv {

// Kernel timing (see sv_trace_* in the C ABI).  When tracing is on, trace_before/trace_after
// record a HIP event on the launch stream immediately before and after the kernel.
bool trace_on();
void trace_before(const char* name, hipStream_t stream);
void trace_after(hipStream_t stream);

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
  const bool tr = trace_on();
  if (tr) trace_before(name, stream);
  const hipError_t err =
      hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shared_bytes,
                      stream);
  if (tr) trace_after(stream);
  return err;
}

template <typename... KArgs, typename... Args>
hipError_t launch_kernel(const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                         hipStream_t stream, Args&&... args) {
  return launch_kernel_shm(name, kernel, grid, block, 0, stream, std::forward<Args>(args)...);
}

}  // namespace sv
