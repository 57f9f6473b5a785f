// Streaming argmax over logit rows: the single HBM sweep of the token-tree and greedy-chain
// verification paths.  Each wave owns one chunk (2048 elements) of one row and writes the
// chunk maximum over non-NaN entries, the lowest index attaining it and whether the chunk holds
// a NaN; the per-row merge happens in the consumer's kernel (merge_row_argmax).

#include <math.h>

#include <atomic>

#include "sv_argmax.h"
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_launch.h"

namespace sv {
namespace {

// Per-load maxima of a lane's elements (load j holds VW of them, widened from its raw 16-byte
// vector).  NANPROP: NaN-propagating maxima (v_maximum3_f32, no canonicalisation of the inputs), so
// a maximum is NaN exactly when its elements hold a NaN; otherwise NaN-ignoring ones (fmaxf).
template <bool NANPROP, typename T, int VW>
__device__ __forceinline__ void load_maxima(const RawChunk<T, VW>& r,
                                            float (&mj)[kElemsPerLane / VW]) {
#pragma unroll
  for (int j = 0; j < kElemsPerLane / VW; ++j) {
    float z[VW];
    if constexpr (VW == 1) {
      z[0] = r.v[j];
    } else {
      unpack<T, VW>(r.v[j], z);
    }
    float v = z[0];
#pragma unroll
    for (int t = 1; t < VW; ++t) v = NANPROP ? __builtin_elementwise_maximum(v, z[t]) : fmaxf(v, z[t]);
    mj[j] = v;
  }
}

// One wave, one loaded chunk -> (max over non-NaN entries, lowest chunk offset holding it
// (INT32_MAX if none), whether the chunk holds a NaN).  The offset is relative to the chunk
// start.  In a row's last chunk the loads past the row repeat its last in-range vector
// (load_raw), so every element past the row is a copy of an element in range at a lower offset:
// it cannot change the maximum, the lowest offset holding it, or the NaN test, and needs no
// masking.  The chunk is taken one load at a time straight from its raw 16-byte vectors (bf16
// pairs widened on the fly), so no widened copy of the chunk is kept.  The per-load maxima are
// first taken NaN-propagating, which also tests for NaN (a lane whose maximum is NaN); only a
// chunk that holds a NaN takes them again NaN-ignoring.  Chunk offsets grow with (load j, lane,
// slot t) in that order, so the lowest offset holding the maximum m is found by ballots instead
// of a per-element search: the first load whose lane maxima include m, the lowest such lane L,
// then the first slot of load j in lane L equal to m (that load is widened again: one compare
// per slot).  -0 equals +0 in these compares, so either sign of a zero maximum finds the lowest
// zero.  A chunk of only NaN has m = NaN and no hit.
template <typename T, int VW>
__device__ __forceinline__ ArgPart argmax_chunk(const RawChunk<T, VW>& r) {
  constexpr int NLD = kElemsPerLane / VW;
  float mj[NLD];
  load_maxima<true>(r, mj);
  float lm = mj[0];
#pragma unroll
  for (int j = 1; j < NLD; ++j) lm = __builtin_elementwise_maximum(lm, mj[j]);
  const bool nan = __any(lm != lm);  // wave-uniform
  float m;
  if (!nan) {
    m = wave_allreduce(lm, [](float a, float b) { return __builtin_elementwise_maximum(a, b); });
  } else {
    load_maxima<false>(r, mj);
    lm = mj[0];
#pragma unroll
    for (int j = 1; j < NLD; ++j) lm = fmaxf(lm, mj[j]);
    m = wave_max(lm);
  }
  int off = INT32_MAX;
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const uint64_t h = __ballot(mj[j] == m);
    if (off == INT32_MAX && h != 0) {  // wave-uniform; taken for the first such load only
      const int L = __builtin_ctzll(h);
      int t_first = 0;
      if constexpr (VW > 1) {
        float z[VW];
        unpack<T, VW>(r.v[j], z);
        t_first = VW;
#pragma unroll
        for (int t = VW - 1; t >= 0; --t)
          if ((__ballot(z[t] == m) >> L) & 1) t_first = t;
      }
      off = chunk_offset<VW>(j, L, t_first);
    }
  }
  return ArgPart{m, off, nan ? 1 : 0, 0};
}

// Workgroup size of the streaming argmax: as the softmax sweep's, except 512 threads for two
// chunks per wave (measured on the 16 x 64 x 32000 bf16 tree workload, about 1% ahead of 256
// threads: 11.91-11.97 against 12.13-12.15 us on one box, 12.02-12.22 against 12.17-12.31 us on
// another; 1024 threads 12.24-12.30 us; with one chunk per wave 256 stays best).
template <typename T, int U>
constexpr int kArgBlock = U == 2 ? 512 : kStreamBlock<T>;

template <typename T, int VW, int U>
__global__ __launch_bounds__((kArgBlock<T, U>), kStreamWavesPerSimd<VW>) void k_argmax_rows(
    const void* logits_v, int64_t V, int64_t nchunk, ArgPart* part, int64_t total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = int64_t(blockIdx.x) * (kArgBlock<T, U> / kWave) + wave_id();
  const T* logits = static_cast<const T*>(logits_v);
  stream_wave<RawChunk<T, VW>, U>(
      gw, total, nchunk, 1,
      [&](const Unit& k, RawChunk<T, VW>& r) {
        load_raw<T, VW>(logits + k.b * V + int64_t(k.c) * kChunk, chunk_valid(V, k.c), lane,
                        r);
      },
      [&](const Unit& k, const RawChunk<T, VW>& r) {
        ArgPart a = argmax_chunk<T, VW>(r);
        a.idx = a.idx == INT32_MAX ? INT32_MAX : a.idx + k.c * kChunk;
        if (lane == 0) part[k.w] = a;
      });
}

// Chunks per wave.  A bf16 launch whose chunks fit one round of resident waves at two chunks per
// wave (but not at one) takes two: every chunk's loads are then issued at the start, with no second
// round of waves waiting for the first to finish.  Otherwise one chunk per wave: finer waves
// shorten the last round's tail.  Measured on bf16 rows: the 16 x 64 x 32000 tree workload
// (16384 chunks, one round at two per wave) 12.6 -> 12.2 us; the 64 x 5 x 128256 greedy workload
// (20160 chunks, 1.23 rounds at two per wave) 14.2 us at one chunk per wave against 15.1 at two.
int resident_waves(int waves_per_simd) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n * 4 * waves_per_simd;  // four SIMDs per compute unit
}

template <typename T, int VW>
hipError_t run(const char* name, const void* logits, int64_t rows, int64_t V, ArgPart* part,
               hipStream_t s) {
  const int64_t nchunk = n_chunks(V);
  const int64_t total = rows * nchunk;
  const int64_t slots = resident_waves(kStreamWavesPerSimd<VW>);
  if constexpr (sizeof(T) == 2 && VW > 1) {  // 4 KiB chunks; an fp32 chunk is already 8 KiB
    constexpr int wpb2 = kArgBlock<T, 2> / kWave;
    if (total > slots && total <= 2 * slots)
      return launch_kernel(name, k_argmax_rows<T, VW, 2>,
                           dim3(unsigned(wave_groups(wave_groups(total, 2), wpb2))),
                           dim3(kArgBlock<T, 2>), s, logits, V, nchunk, part, total);
  }
  constexpr int wpb = kArgBlock<T, 1> / kWave;
  return launch_kernel(name, k_argmax_rows<T, VW, 1>, dim3(unsigned(wave_groups(total, wpb))),
                       dim3(kArgBlock<T, 1>), s, logits, V, nchunk, part, total);
}

}  // namespace

hipError_t launch_argmax_rows(const char* name, const void* logits, sv_dtype dtype, bool vec,
                              int64_t rows, int64_t V, ArgPart* part, hipStream_t s) {
  if (dtype == SV_F32)
    return vec ? run<float, 4>(name, logits, rows, V, part, s)
               : run<float, 1>(name, logits, rows, V, part, s);
  return vec ? run<uint16_t, 8>(name, logits, rows, V, part, s)
             : run<uint16_t, 1>(name, logits, rows, V, part, s);
}

}  // namespace sv
