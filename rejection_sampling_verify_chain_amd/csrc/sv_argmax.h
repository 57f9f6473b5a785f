// Argmax partials of logit rows: the chunk partial record, its merge order, and the launcher of
// the streaming argmax kernel (sv_argmax.hip).  Shared by the token-tree and greedy-chain
// verification paths.
#pragma once

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

// Streams rows [0, rows) of `logits` (contiguous rows of V elements of dtype; vec: the
// 16-byte-load path is legal) and writes one ArgPart per (row, chunk) to part[row * nchunk + c].
// The launch is named `name` for kernel timing.
hipError_t launch_argmax_rows(const char* name, const void* logits, sv_dtype dtype, bool vec,
                              int64_t rows, int64_t V, ArgPart* part, hipStream_t stream);

// (value, index) order of the argmax: larger value first, then lower index.
__device__ __forceinline__ bool arg_better(float v, int32_t i, float bv, int32_t bi) {
  return v > bv || (v == bv && i < bi);
}

// One wave merges the chunk partials of one logit row: the row's argmax (lowest index among
// equal maxima) and whether the row holds a NaN.  Lanes take chunks, all loads of a batch in
// flight together, then a butterfly reduction with the argmax order.

__device__ __forceinline__ void merge_row_argmax(const ArgPart* pp, int64_t nchunk, int lane,
                                                 int32_t* g, int* nan) {
  float best = -INFINITY;
  int32_t bidx = INT32_MAX;
  int anynan = 0;
  for (int64_t base = 0; base < nchunk; base += int64_t(kWave) * kMergeBatch) {
    ArgPart r[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int64_t c = base + i * kWave + lane;
      r[i] = c < nchunk ? pp[c] : ArgPart{-INFINITY, INT32_MAX, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (arg_better(r[i].v, r[i].idx, best, bidx)) {
        best = r[i].v;
        bidx = r[i].idx;
      }
      anynan |= r[i].nan;
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, kWave);
    const int32_t oi = __shfl_xor(bidx, o, kWave);
    if (arg_better(ov, oi, best, bidx)) {
      best = ov;
      bidx = oi;
    }
  }
  *g = bidx == INT32_MAX ? 0 : bidx;
  *nan = __any(anynan);
}

}  // namespace sv
