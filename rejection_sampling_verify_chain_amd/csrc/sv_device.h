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
// wave that owns chunk c issues kElemsPerLane / VW loads of VW elements each;
// load j covers the VW elements starting at chunk offset (j * 64 + lane) * VW,
// so every load instruction reads 64 * VW consecutive elements (1 KiB for the
// 16-byte vector forms).  Element (j, t) of a lane lands in z[j * VW + t]; the
// chunk's element order is (j, lane, t) lexicographic.  Elements at or beyond V
// are not read and are set to -inf.
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

// A lane's share of chunk c as loaded: the raw 16-byte vectors (VW > 1), or the widened
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

template <typename T, int VW>
__device__ __forceinline__ void load_raw(const T* __restrict__ row, int64_t V, int64_t c, int lane,
                                         RawChunk<T, VW>& r) {
  const int64_t c0 = c * kChunk;
  if constexpr (VW == 1) {
#pragma unroll
    for (int j = 0; j < kElemsPerLane; ++j) {
      const int64_t e = c0 + j * kWave + lane;
      r.v[j] = e < V ? widen(__builtin_nontemporal_load(&row[e])) : -INFINITY;
    }
  } else {
    using VT = typename Vec<T, VW>::type;
    const VT* vrow = reinterpret_cast<const VT*>(row);
    const int64_t nvec = V / VW;
    const int64_t v0 = c0 / VW;
#pragma unroll
    for (int j = 0; j < kElemsPerLane / VW; ++j) {
      const int64_t vi = v0 + j * kWave + lane;
      if (vi < nvec) r.v[j] = __builtin_nontemporal_load(&vrow[vi]);
    }
  }
}

// z[j * VW + t] = element (j, t) of the lane's share, -inf beyond V.
template <typename T, int VW>
__device__ __forceinline__ void unpack_chunk(const RawChunk<T, VW>& r, int64_t V, int64_t c,
                                             int lane, float (&z)[kElemsPerLane]) {
  if constexpr (VW == 1) {
#pragma unroll
    for (int j = 0; j < kElemsPerLane; ++j) z[j] = r.v[j];
  } else {
    const int64_t nvec = V / VW;
    const int64_t v0 = c * kChunk / VW;
#pragma unroll
    for (int j = 0; j < kElemsPerLane / VW; ++j) {
      if (v0 + j * kWave + lane < nvec) {
        unpack<T, VW>(r.v[j], &z[j * VW]);
      } else {
#pragma unroll
        for (int t = 0; t < VW; ++t) z[j * VW + t] = -INFINITY;
      }
    }
  }
}

// The lane's share of chunk c, widened: z[j * VW + t] holds element (j, t).
template <typename T, int VW>
__device__ __forceinline__ void load_chunk(const T* __restrict__ row, int64_t V, int64_t c, int lane,
                                           float (&z)[kElemsPerLane]) {
  RawChunk<T, VW> r;
  load_raw<T, VW>(row, V, c, lane, r);
  unpack_chunk<T, VW>(r, V, c, lane, z);
}

// ---------------------------------------------------------------------------- wave collectives
// Butterfly (xor) reductions: every lane ends with the same, bitwise identical value.

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}

// Inclusive prefix sum over the lanes of a wave (Hillis-Steele).
__device__ __forceinline__ double wave_inclusive_scan(double v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ double wave_broadcast(double v, int src) { return __shfl(v, src, kWave); }

// (row, chunk) units one wave of a streaming kernel takes: its loads for all of them are issued
// together, 8 KiB per wave (one fp32 chunk, two bf16 chunks), which keeps enough bytes in
// flight per compute unit for HBM to stay saturated while other waves compute.
template <typename T>
constexpr int units_per_wave() {
  return 4 / int(sizeof(T));
}

// Index of the calling wave within its workgroup, as a wave-uniform (scalar) value: index
// arithmetic derived from it runs on the scalar unit instead of every lane.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kWave);
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
