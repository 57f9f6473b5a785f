// Streaming-read ceiling: a kernel that only reads, the way the streaming kernels read logits
// (one 8 KiB piece per wave as eight 16-byte nontemporal loads per lane, 1024-thread
// workgroups, 8 waves per SIMD), so that the verify kernels' HBM rates can be set beside the
// rate of a plain read of the same size, measured in the same run.  Measurement support only.

#include <stdint.h>

#include "sv_device.h"
#include "sv_internal.h"
#include "sv_launch.h"

namespace sv {
namespace {


// Each workgroup writes the XOR of every word it read (so no load can be dropped).
__global__ __launch_bounds__(kProbeBlock, 8) void k_read_probe(const u32x4_t* __restrict__ src,
                                                               int64_t n16, uint32_t* out) {
  __shared__ uint32_t part[kProbeBlock / kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_id();
  const int64_t base = (int64_t(blockIdx.x) * (kProbeBlock / kWave) + wave) * kProbeWave16;
  u32x4_t v[kProbeLoads];
#pragma unroll
  for (int j = 0; j < kProbeLoads; ++j) {
    const int64_t i = base + int64_t(j) * kWave + lane;
    v[j] = i < n16 ? __builtin_nontemporal_load(&src[i]) : u32x4_t{0u, 0u, 0u, 0u};
  }
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < kProbeLoads; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  x = uint32_t(wave_allreduce(int(x), [](int a, int b) { return a ^ b; }));
  if (lane == 0) part[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < kProbeBlock / kWave; ++w) y ^= part[w];
    out[blockIdx.x] = y;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* out, hipStream_t s) {
  return launch_kernel("read_probe", k_read_probe, dim3(unsigned(read_probe_groups(bytes))),
                       dim3(kProbeBlock), s, static_cast<const u32x4_t*>(src), bytes / 16, out);
}

}  // namespace sv
