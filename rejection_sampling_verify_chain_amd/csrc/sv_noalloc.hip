// Static device scratch of the entry point that allocates nothing (sv_verify_chain_noalloc).
//
// The chain kernels take their workspace (chunk partials, row statistics, decisions, residual
// masses) from this file-scope array instead of a caller buffer.  Every GPU the library runs on
// holds its own copy, SV_NOALLOC_SCRATCH_BYTES large, from the first kernel launch of the process
// until it ends.  In host code `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device with hipGetSymbolAddress and only that address is ever
// handed to a kernel.  Calls that overlap in time on one GPU share the array and race; the
// chain path writes every entry it reads within a call, so nothing needs clearing between calls.

#include <hip/hip_runtime.h>

#include <atomic>

#include "sv_internal.h"

static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace sv {
namespace {

constexpr int kMaxDevices = 256;
// Device address of each GPU's copy of `scratch`, or nullptr before its first lookup.  Two
// threads that look a device up at once store the same address.
std::atomic<void*> g_scratch[kMaxDevices];

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace sv
