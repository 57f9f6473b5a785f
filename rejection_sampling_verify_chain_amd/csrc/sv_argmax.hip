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
// offset is relative to the chunk start.  Each lane finds its lowest slot i = j * VW + t holding
// the maximum (slots increase with the chunk offset inside a lane), then a wave minimum over
// the offsets gives the chunk's lowest.  Branch-free; a chunk of only -inf finds its first
// in-range -inf element, a chunk of only NaN none.
template <int VW, bool TAIL>
__device__ __forceinline__ ArgPart argmax_chunk(const float (&z)[kElemsPerLane], int nvalid,
                                                int lane) {
  float m = -INFINITY;
  bool nan = false;
#pragma unroll
  for (int i = 0; i < kElemsPerLane; ++i) {
    m = fmaxf(m, z[i]);  // NaN never wins
    nan |= (z[i] != z[i]);
  }
  m = wave_max(m);
  int slot = kElemsPerLane;
#pragma unroll
  for (int i = kElemsPerLane - 1; i >= 0; --i) {
    bool hit = z[i] == m;
    if (TAIL) hit = hit && chunk_offset<VW>(i / VW, lane, i % VW) < nvalid;
    slot = hit ? i : slot;
  }
  const int off = slot < kElemsPerLane ? chunk_offset<VW>(slot / VW, lane, slot % VW) : INT32_MAX;
  return ArgPart{m, wave_min(off), __any(nan) ? 1 : 0, 0};
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
        ArgPart a = nvalid == kChunk ? argmax_chunk<VW, false>(z, nvalid, lane)
                                     : argmax_chunk<VW, true>(z, nvalid, lane);
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
  return launch_kernel(name, k_argmax_rows<T, VW>, dim3(unsigned((total + wpb - 1) / wpb)),
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
