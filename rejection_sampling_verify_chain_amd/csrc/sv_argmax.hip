// Streaming argmax over logit rows: the single HBM sweep of the token-tree and greedy-chain
// verification paths.  Each wave owns one chunk (2048 elements) of one row and writes the
// chunk maximum over non-NaN entries, the lowest index attaining it and whether the chunk holds
// a NaN; the per-row merge happens in the consumer's kernel (merge_row_argmax).

#include <math.h>

#include "sv_argmax.h"
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_launch.h"

namespace sv {
namespace {

// One wave, one loaded chunk whose first nvalid elements exist -> (max over non-NaN entries,
// lowest chunk offset holding it (INT32_MAX if none), whether the chunk holds a NaN).  The
// offset is relative to the chunk start.  Chunk offsets grow with (load j, lane, slot t) in
// that order, so the lowest offset holding the maximum m is found by ballots instead of a
// per-element search: the first load whose lane maxima include m, the lowest such lane L, then
// the first slot of load j in lane L equal to m (one compare per load, one per slot of the
// found load).  Elements past nvalid are -inf and come after every element in range, so in a
// row's last chunk a hit at or past nvalid means none in range.  A chunk of only NaN has m =
// NaN and no hit.
template <int VW, bool TAIL>
__device__ __forceinline__ ArgPart argmax_chunk(const float (&z)[kElemsPerLane], int nvalid) {
  constexpr int NLD = kElemsPerLane / VW;
  float mj[NLD];
  bool nan = false;
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    float v = z[j * VW];
#pragma unroll
    for (int t = 1; t < VW; ++t) v = fmaxf(v, z[j * VW + t]);  // NaN never wins
    mj[j] = v;
  }
#pragma unroll
  for (int i = 0; i < kElemsPerLane; ++i) nan |= (z[i] != z[i]);
  float lm = mj[0];
#pragma unroll
  for (int j = 1; j < NLD; ++j) lm = fmaxf(lm, mj[j]);
  const float m = wave_max(lm);
  int off = INT32_MAX;
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const uint64_t h = __ballot(mj[j] == m);
    if (off == INT32_MAX && h != 0) {  // wave-uniform; taken for the first such load only
      const int L = __builtin_ctzll(h);
      int t_first = VW;
#pragma unroll
      for (int t = VW - 1; t >= 0; --t)
        if ((__ballot(z[j * VW + t] == m) >> L) & 1) t_first = t;
      off = chunk_offset<VW>(j, L, t_first);
    }
  }
  if (TAIL && off >= nvalid) off = INT32_MAX;
  return ArgPart{m, off, __any(nan) ? 1 : 0, 0};
}

template <typename T, int VW>
__global__ __launch_bounds__(kStreamBlock<T>, kStreamWavesPerSimd<VW>) void k_argmax_rows(
    const void* logits_v, int64_t V, int64_t nchunk, ArgPart* part, int64_t total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = int64_t(blockIdx.x) * (kStreamBlock<T> / kWave) + wave_id();
  const T* logits = static_cast<const T*>(logits_v);
  stream_wave<RawChunk<T, VW>, 1>(
      gw, total, nchunk, 1,
      [&](const Unit& k, RawChunk<T, VW>& r) {
        load_raw<T, VW>(logits + k.b * V + int64_t(k.c) * kChunk, chunk_valid(V, k.c), lane,
                        r);
      },
      [&](const Unit& k, const RawChunk<T, VW>& r) {
        const int nvalid = chunk_valid(V, k.c);
        float z[kElemsPerLane];
        unpack_chunk<T, VW>(r, nvalid, lane, z);
        ArgPart a = nvalid == kChunk ? argmax_chunk<VW, false>(z, nvalid)
                                     : argmax_chunk<VW, true>(z, nvalid);
        a.idx = a.idx == INT32_MAX ? INT32_MAX : a.idx + k.c * kChunk;
        if (lane == 0) part[k.w] = a;
      });
}

template <typename T, int VW>
hipError_t run(const char* name, const void* logits, int64_t rows, int64_t V, ArgPart* part,
               hipStream_t s) {
  // One chunk per wave: at 64 registers the argmax runs 8 waves per SIMD, which measured
  // faster than two bf16 chunks per wave at the lower occupancy their registers allow.
  const int64_t nchunk = n_chunks(V);
  const int64_t total = rows * nchunk;
  constexpr int wpb = kStreamBlock<T> / kWave;
  return launch_kernel(name, k_argmax_rows<T, VW>, dim3(unsigned(wave_groups(total, wpb))),
                       dim3(kStreamBlock<T>), s, logits, V, nchunk, part, total);
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
