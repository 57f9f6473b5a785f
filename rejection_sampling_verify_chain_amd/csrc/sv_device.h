// Device-side building blocks: exact logit widening, chunk loads, wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_internal.h"

namespace sv {

// ---------------------------------------------------------------------------- widening

// bf16 is the upper half of an fp32 word: widening is a 16-bit shift, exact.
__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// ---------------------------------------------------------------------------- chunk loads
//
// A chunk is kChunk consecutive elements of one logit row.  Lane `lane` of the
// wave that owns a chunk issues kElemsPerLane / VW loads of VW elements each;
// load j covers the VW elements starting at chunk offset (j * 64 + lane) * VW,
// so every load instruction reads 64 * VW consecutive elements (1 KiB for the
// 16-byte vector forms).  Element (j, t) of a lane lands in z[j * VW + t]; the
// chunk's element order is (j, lane, t) lexicographic.  Only the first `nvalid`
// elements of a chunk exist (kChunk for every chunk but a row's last); the
// others are not read and are set to -inf.
//
// VW = 4 (fp32) and VW = 8 (bf16) are 16-byte loads and require a 16-byte
// aligned row start and V % VW == 0 (checked on the host); VW = 1 reads one
// element per load and has no alignment requirement.  Logits are streamed once,
// so the loads carry the nontemporal hint (measured: the fp32 sweep of 2.3 GB
// goes from 6.3 to 6.9 TB/s).

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <typename T, int VW>
struct Vec;
template <>
struct Vec<float, 4> {
  using type = f32x4_t;
};
template <>
struct Vec<uint16_t, 8> {
  using type = u32x4_t;
};

template <typename T, int VW>
__device__ __forceinline__ void unpack(const typename Vec<T, VW>::type& v, float* out);

template <>
__device__ __forceinline__ void unpack<float, 4>(const f32x4_t& v, float* out) {
  out[0] = v.x;
  out[1] = v.y;
  out[2] = v.z;
  out[3] = v.w;
}

template <>
__device__ __forceinline__ void unpack<uint16_t, 8>(const u32x4_t& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Chunk offset (in elements) of element (j, t) of `lane`.
template <int VW>
__device__ __forceinline__ int chunk_offset(int j, int lane, int t) {
  return (j * kWave + lane) * VW + t;
}

// Elements of chunk c of a row of V that lie inside the row (wave-uniform).
__device__ __forceinline__ int chunk_valid(int64_t V, int64_t c) {
  const int64_t r = V - c * kChunk;
  return r >= kChunk ? kChunk : int(r);
}

// A lane's share of a chunk as loaded: the raw 16-byte vectors (VW > 1), or the widened
// elements (VW == 1).  Widening the vector forms into floats is left to unpack_chunk, so that a
// wave can hold several chunks in flight at 4 (fp32) or 2 (bf16) elements per register.
template <typename T, int VW>
struct RawChunk {
  typename Vec<T, VW>::type v[kElemsPerLane / VW];
};
template <typename T>
struct RawChunk<T, 1> {
  float v[kElemsPerLane];
};

// Issue the loads of the chunk starting at `base` (nvalid >= 1 elements in range).  Every
// lane issues the same kElemsPerLane / VW loads whatever nvalid is: in a row's last chunk the
// loads past the row are redirected to its last in-range vector (the same cache line, so no
// extra HBM traffic) and unpack_chunk masks them.  A fixed load count keeps the compiler's
// wait counting exact, so a wave can reduce one chunk while the next one's loads are in flight.
template <typename T, int VW>
__device__ __forceinline__ void load_raw(const T* __restrict__ base, int nvalid, int lane,
                                         RawChunk<T, VW>& r) {
  if constexpr (VW == 1) {
#pragma unroll
    for (int j = 0; j < kElemsPerLane; ++j) {
      const int e = j * kWave + lane;
      r.v[j] = widen(__builtin_nontemporal_load(&base[e < nvalid ? e : nvalid - 1]));
    }
  } else {
    using VT = typename Vec<T, VW>::type;
    const VT* vb = reinterpret_cast<const VT*>(base);
    if (nvalid == kChunk) {
#pragma unroll
      for (int j = 0; j < kElemsPerLane / VW; ++j)
        r.v[j] = __builtin_nontemporal_load(&vb[j * kWave + lane]);
    } else {
      const int last = nvalid / VW - 1;  // nvalid is a multiple of VW on this path
#pragma unroll
      for (int j = 0; j < kElemsPerLane / VW; ++j)
        r.v[j] = __builtin_nontemporal_load(&vb[min(j * kWave + lane, last)]);
    }
  }
}

// z[j * VW + t] = element (j, t) of the lane's share, -inf beyond the row.
template <typename T, int VW>
__device__ __forceinline__ void unpack_chunk(const RawChunk<T, VW>& r, int nvalid, int lane,
                                             float (&z)[kElemsPerLane]) {
  if constexpr (VW == 1) {
#pragma unroll
    for (int j = 0; j < kElemsPerLane; ++j) z[j] = r.v[j];
  } else {
#pragma unroll
    for (int j = 0; j < kElemsPerLane / VW; ++j) unpack<T, VW>(r.v[j], &z[j * VW]);
  }
  if (nvalid != kChunk) {
#pragma unroll
    for (int j = 0; j < kElemsPerLane / VW; ++j) {
      const bool in = (j * kWave + lane) * VW < nvalid;
#pragma unroll
      for (int t = 0; t < VW; ++t) z[j * VW + t] = in ? z[j * VW + t] : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------- streaming waves
//
// The streaming kernels (softmax partials, argmax partials) give each wave one chunk of logits
// to load at once (8 KiB of fp32, 4 KiB of bf16), all its loads issued before it is reduced.
// Units are the chunks of all rows in row-major order, unit w = row * nchunk + c (a row's last
// chunk may be partial), rows coming in groups of R (the rows of one sequence).  Measured
// alternatives that lost: a persistent grid-stride loop with the next unit's loads in flight
// (slower at every size here), moving the partial chunks into waves of their own (2% slower on
// a 2.3 GB fp32 sweep), and two bf16 chunks per wave (6-7% slower on the 148 MB bf16 sweeps).

// Units (chunks) a wave takes.
template <typename T>
constexpr int kUnitsPerWave = 1;

// Workgroup size of the streaming kernels (measured): 1024 threads for fp32 logits, 256 for bf16.
template <typename T>
constexpr int kStreamBlock = sizeof(T) == 4 ? 1024 : 256;
static_assert(kStreamBlock<uint16_t> <= kMaxBlock && kStreamBlock<float> <= kMaxBlock,
              "the C ABI's launch limits assume workgroups of at most kMaxBlock threads");

// Occupancy the vector-load streaming kernels are compiled for: 8 waves per SIMD (at most 64
// VGPRs, reached without spills).  The one-element-load forms (unaligned rows) are left
// unconstrained.
template <int VW>
constexpr int kStreamWavesPerSimd = VW > 1 ? 8 : 1;

struct Unit {
  int64_t w;  // unit index
  int64_t b;  // group (row / R)
  int32_t j;  // row within the group
  int32_t c;  // chunk within the row
};

__device__ __forceinline__ Unit unit_at(int64_t w, int64_t nchunk, int R) {
  const int64_t row = w / nchunk;
  Unit k;
  k.w = w;
  k.c = int32_t(w - row * nchunk);
  k.b = row / R;
  k.j = int32_t(row - k.b * R);
  return k;
}

__device__ __forceinline__ Unit unit_after(Unit k, int64_t nchunk, int R) {
  k.w += 1;
  if (++k.c == nchunk) {
    k.c = 0;
    if (++k.j == R) {
      k.j = 0;
      k.b += 1;
    }
  }
  return k;
}

// Runs wave gw of a streaming kernel over `total` units: issue(unit, raw) starts a unit's loads
// and proc(unit, raw) reduces it.  Wave-uniform control flow.
template <typename Raw, int U, typename IssueFn, typename ProcFn>
__device__ __forceinline__ void stream_wave(int64_t gw, int64_t total, int64_t nchunk, int R,
                                            IssueFn issue, ProcFn proc) {
  static_assert(U == 1 || U == 2, "one or two units per wave");
  const int64_t w0 = gw * U;
  if (w0 >= total) return;
  const Unit k0 = unit_at(w0, nchunk, R);
  Raw r0;
  issue(k0, r0);
  if constexpr (U == 2) {
    if (w0 + 1 < total) {
      const Unit k1 = unit_after(k0, nchunk, R);
      Raw r1;
      issue(k1, r1);
      proc(k0, r0);
      proc(k1, r1);
      return;
    }
  }
  proc(k0, r0);
}

// Per-lane batch of the partial merges: a lane takes kMergeBatch partials of a row at a time
// with all their loads in flight, so rows of up to 64 * kMergeBatch chunks are read at once.
constexpr int kMergeBatch = 4;

// ---------------------------------------------------------------------------- wave collectives
// All-lane reductions over a full wave (all 64 lanes active).  Inside each row of 16 lanes four
// DPP steps combine partners (quad swaps, then the half-row and row mirrors), leaving the row's
// result in all 16 lanes; the four row results are read out with readlane and combined in one
// fixed order.  Every lane ends with the same, bitwise identical value (each DPP step combines
// two equal-shaped halves, and the operations are commutative).  DPP runs in the vector ALU;
// the cross-lane shuffle it replaces goes through the LDS crossbar once per step.

// dpp_ctrl values: quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror.
constexpr int kDppQuadSwap1 = 0xB1;
constexpr int kDppQuadSwap2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = uint32_t(dpp<CTRL>(int(uint32_t(u)))), hi = uint32_t(dpp<CTRL>(int(uint32_t(u >> 32))));
  return __longlong_as_double((uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ int lane_read(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_read(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ int64_t lane_read(int64_t v, int l) {
  const uint64_t u = uint64_t(v);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u >> 32)), l));
  return int64_t((uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ double lane_read(double v, int l) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u >> 32)), l));
  return __longlong_as_double((uint64_t(hi) << 32) | lo);
}

template <typename T, typename Op>
__device__ __forceinline__ T wave_allreduce(T v, Op op) {
  v = op(v, dpp<kDppQuadSwap1>(v));
  v = op(v, dpp<kDppQuadSwap2>(v));
  v = op(v, dpp<kDppHalfMirror>(v));
  v = op(v, dpp<kDppMirror>(v));
  return op(op(lane_read(v, 0), lane_read(v, 16)), op(lane_read(v, 32), lane_read(v, 48)));
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_allreduce(v, [](float a, float b) { return fmaxf(a, b); });
}

__device__ __forceinline__ double wave_sum(double v) {
  return wave_allreduce(v, [](double a, double b) { return a + b; });
}

__device__ __forceinline__ int wave_min(int v) {
  return wave_allreduce(v, [](int a, int b) { return min(a, b); });
}

__device__ __forceinline__ int wave_max_int(int v) {
  return wave_allreduce(v, [](int a, int b) { return max(a, b); });
}

// Row shift right by N lanes inside each row of 16 lanes (dpp_ctrl row_shr:N); a lane whose
// source would lie before its row's first lane reads 0.
template <int N>
__device__ __forceinline__ double dpp_shr_zero(double v) {
  static_assert(N >= 1 && N <= 15, "row_shr takes 1..15");
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(u)), 0x110 + N, 0xF, 0xF, true));
  const uint32_t hi =
      uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(u >> 32)), 0x110 + N, 0xF, 0xF, true));
  return __longlong_as_double((uint64_t(hi) << 32) | lo);
}

// Inclusive prefix sum over the lanes of a wave, fp64, in the vector ALU: four DPP shift-and-add
// steps (1, 2, 4, 8 lanes) give each lane the prefix inside its row of 16; the totals of rows 0-2
// (lanes 15, 31, 47) are then read out and added to the later rows in one fixed order.  Every
// caller sums its lanes this way, so a sum recomputed by another kernel has the same bits.
__device__ __forceinline__ double wave_inclusive_scan(double v, int lane) {
  v += dpp_shr_zero<1>(v);
  v += dpp_shr_zero<2>(v);
  v += dpp_shr_zero<4>(v);
  v += dpp_shr_zero<8>(v);
  const double r0 = lane_read(v, 15), r1 = lane_read(v, 31), r2 = lane_read(v, 47);
  const int row = lane >> 4;
  const double off = row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2;
  return row == 0 ? v : v + off;
}

// The value of lane `src` (wave-uniform) in every lane.
__device__ __forceinline__ double wave_broadcast(double v, int src) { return lane_read(v, src); }

// Index of the calling wave within its workgroup, as a wave-uniform (scalar) value: index
// arithmetic derived from it runs on the scalar unit instead of every lane.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
}

// Wave-uniform read of data that no wave of the running kernel writes, through the scalar data
// cache (a scalar load, counted apart from the vector loads, so waiting for it never waits for
// chunk loads in flight).  Records of 16 bytes (the workspace's partials, statistics and
// decisions) are read as four dwords and reinterpreted.
template <typename T>
__device__ __forceinline__ T uniform_load(const T* p, int64_t i) {
  if constexpr (sizeof(T) == 16) {
    static_assert(alignof(T) == 16, "16-byte records must be 16-byte aligned");
    const u32x4_t v = ((const __attribute__((address_space(4))) u32x4_t*)p)[i];
    return __builtin_bit_cast(T, v);
  } else {
    return ((const __attribute__((address_space(4))) T*)p)[i];
  }
}

// 2^x on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The temperature used for arithmetic: T itself when finite and positive, else 1.  A sequence
// with an invalid T is reported and takes the fallback result; substituting 1 keeps its row
// statistics meaningful, so the logit checks (NaN, +inf, all -inf) do not depend on T.
__device__ __forceinline__ float effective_temperature(float T) {
  return (T > 0.0f && T < INFINITY) ? T : 1.0f;
}

// log2(e) / T in fp32, correctly rounded; every kernel forms it the same way so that
// per-element terms recomputed in a later kernel are bitwise identical.  Clamped to the
// largest finite float so that a tiny T gives (z - m) * k = 0 (not NaN) at the maximum.
__device__ __forceinline__ float log2e_over_t(float T) {
  return fminf(1.4426950408889634f / T, 3.40282347e38f);
}

}  // namespace sv
