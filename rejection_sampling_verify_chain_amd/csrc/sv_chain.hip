// Chain verification kernels (speculative sampling, target side).
//
// Source: "論文解説: Speculative Sampling — ドラフトモデルによるLLMデコード高速化"
// (0h-n0.github.io explainer of arXiv:2302.01318): Step 2 (ステップ2) gives the
// gamma+1 target distributions of one pass, Step 3 (ステップ3) the accept test
// min(1, p/q) applied in order with a cut at the first rejection, the modified
// rejection sampling section (修正付き棄却サンプリング) the residual
// norm(max(0, p - q)), and the expected-speedup section the (gamma+1)-th token
// of a fully accepted round.
//
// Pipeline (all on the caller's stream, no host synchronisation):
//   1. rowstats  one wave per (row, chunk) of every logit row, target and draft:
//                chunk max m_c and S_c = sum exp((z - m_c)/T) (fp32 terms, fp64 sum).
//                This is the single HBM sweep over all B*(2*gamma+1)*V logits.
//   2. decide    one workgroup per sequence: merges the chunk partials into the
//                row max and normaliser, evaluates p_i(x_i), q_i(x_i) in fp64 (one
//                lane per position), takes the accept bits with a ballot and the
//                cut k = number of leading ones.
//   3. residual  one wave per (sequence, chunk) of rejecting sequences: chunk mass
//                W_c = sum max(0, p_k - q_k) over target and draft row k.
//   4. draw      one wave per sequence: running sum over chunk masses (residual
//                W_c, or the bonus row's p mass from step 1), locate the chunk
//                holding u*W, re-scan that chunk in token order, write y.

#include <math.h>

#include "sv_device.h"
#include "sv_internal.h"
#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

template <typename T>
__device__ __forceinline__ const T* chain_row(const T* tgt, const T* drf, int64_t b, int gamma,
                                              int j, int64_t V) {
  // Virtual row j of sequence b: j <= gamma is target row j, else draft row j - gamma - 1.
  return j <= gamma ? tgt + (b * (gamma + 1) + j) * V
                    : drf + (b * gamma + (j - gamma - 1)) * V;
}

// exp((z - m) / T) for an element of a chunk whose maximum is m, as 2^((z - m) * log2e/T).
__device__ __forceinline__ float softmax_term(float z, float m, float k) {
  return hw_exp2((z - m) * k);
}

// Factor taking a chunk-local term to a normalised probability: exp((m_c - M)/T) / S.
__device__ __forceinline__ double chunk_scale(float mc, const RowStat& st, double Td) {
  if (mc == -INFINITY) return 0.0;
  return exp((double(mc) - double(st.m)) / Td) / st.s;
}

// Residual weight max(0, p(x) - q(x)) at one token, from the chunk-local terms.
__device__ __forceinline__ double residual_term(float zt, float zd, float mt, float md, float k,
                                                double A, double Bq) {
  const double pt = A > 0.0 ? double(softmax_term(zt, mt, k)) * A : 0.0;
  const double qd = Bq > 0.0 ? double(softmax_term(zd, md, k)) * Bq : 0.0;
  const double d = pt - qd;
  return d > 0.0 ? d : 0.0;
}

// ------------------------------------------------------------------------------------ 1. rowstats
template <typename T, int VW>
__global__ __launch_bounds__(kBlock) void k_chain_rowstats(const T* __restrict__ tgt,
                                                           const T* __restrict__ drf,
                                                           const float* __restrict__ temp,
                                                           int gamma, int64_t V, int64_t nchunk,
                                                           int64_t total_chunks,
                                                           RowPart* __restrict__ part) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t w = int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x / kWave);
  if (w >= total_chunks) return;  // wave-uniform
  const int R = 2 * gamma + 1;
  const int64_t row = w / nchunk;
  const int64_t c = w - row * nchunk;
  const int64_t b = row / R;
  const int j = int(row - b * R);

  float z[kElemsPerLane];
  load_chunk<T, VW>(chain_row(tgt, drf, b, gamma, j, V), V, c, lane, z);

  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kElemsPerLane; ++i) m = fmaxf(m, z[i]);
  m = wave_max(m);

  double s;
  if (m == -INFINITY) {
    // Only -inf (or NaN) in this chunk: its mass is zero unless a NaN poisons the row.
    bool nan = false;
#pragma unroll
    for (int i = 0; i < kElemsPerLane; ++i) nan |= (z[i] != z[i]);
    s = __any(nan) ? NAN : 0.0;
  } else {
    const float k = log2e_over_t(effective_temperature(temp[b]));
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < kElemsPerLane; ++i) acc[i & 3] += double(softmax_term(z[i], m, k));
    s = wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
  }
  if (lane == 0) part[w] = RowPart{m, 0, s};
}

// ------------------------------------------------------------------------------------ 2. decide
template <typename T>
__global__ __launch_bounds__(kBlock) void k_chain_decide(
    const T* __restrict__ tgt, const T* __restrict__ drf, const int32_t* __restrict__ toks,
    const float* __restrict__ uni, const float* __restrict__ temp, int gamma, int64_t V,
    int64_t nchunk, const RowPart* __restrict__ part, RowStat* __restrict__ rowstat,
    SeqDecision* __restrict__ seq, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_nacc, float* __restrict__ out_p, float* __restrict__ out_q,
    int32_t* __restrict__ out_status) {
  __shared__ RowStat st[2 * kMaxGamma + 1];
  const int64_t b = blockIdx.x;
  const int R = 2 * gamma + 1;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const float tb = temp[b];
  const float te = effective_temperature(tb);
  const double Td = te;

  // Merge chunk partials: M = max_c m_c, S = sum_c S_c exp((m_c - M)/T).
  for (int j = wave; j < R; j += kWavesPerBlock) {
    const RowPart* pp = part + (b * R + j) * nchunk;
    float m = -INFINITY;
    for (int64_t c = lane; c < nchunk; c += kWave) m = fmaxf(m, pp[c].m);
    m = wave_max(m);
    double s = 0.0;
    const bool finite_max = (m > -INFINITY) && (m < INFINITY);
    if (finite_max) {
      for (int64_t c = lane; c < nchunk; c += kWave) {
        const RowPart q = pp[c];
        const double f = q.m == -INFINITY ? 0.0 : exp((double(q.m) - double(m)) / Td);
        s += q.s * f;  // a NaN partial survives the zero factor
      }
    }
    s = wave_sum(s);
    const int valid = finite_max && (s > 0.0) && (s < INFINITY);
    if (lane == 0) {
      st[j] = RowStat{m, valid, s};
      rowstat[b * R + j] = st[j];
    }
  }
  __syncthreads();
  if (wave != 0) return;

  int status = 0;
  if (!(tb > 0.0f && tb < INFINITY)) status |= SV_ROW_BAD_TEMPERATURE;
  bool bad = false;
  for (int i = lane; i <= gamma; i += kWave) {
    const float u = uni[b * (gamma + 1) + i];
    bad |= !(u >= 0.0f && u < 1.0f);
  }
  if (__any(bad)) status |= SV_ROW_BAD_UNIFORM;
  int x = 0;
  bad = false;
  if (lane < gamma) {
    x = toks[b * gamma + lane];
    bad = (x < 0) || (int64_t(x) >= V);
  }
  if (__any(bad)) status |= SV_ROW_TOKEN_RANGE;
  bad = false;
  for (int j = lane; j < R; j += kWave) bad |= !st[j].valid;
  if (__any(bad)) status |= SV_ROW_NONFINITE;

  const bool fallback = (status & (SV_ROW_TOKEN_RANGE | SV_ROW_NONFINITE |
                                   SV_ROW_BAD_TEMPERATURE | SV_ROW_BAD_UNIFORM)) != 0;
  int k = 0;
  bool accept = false;
  if (!fallback) {
    double p = 0.0, q = 0.0;
    if (lane < gamma) {
      const RowStat a = st[lane];
      const RowStat d = st[gamma + 1 + lane];
      const double zt = widen(chain_row(tgt, drf, b, gamma, lane, V)[x]);
      const double zd = widen(chain_row(tgt, drf, b, gamma, gamma + 1 + lane, V)[x]);
      p = exp((zt - double(a.m)) / Td) / a.s;
      q = exp((zd - double(d.m)) / Td) / d.s;
      const double u = uni[b * (gamma + 1) + lane];
      if (q > 0.0) {
        accept = u < fmin(1.0, p / q);
      } else {
        accept = (p > 0.0) && (u < 1.0);  // ratio +inf; p = q = 0 rejects
      }
      if (out_p) out_p[b * gamma + lane] = float(p);
      if (out_q) out_q[b * gamma + lane] = float(q);
    }
    // Cut at the first rejection: k = number of leading ones of the accept mask.
    const uint64_t rej = ~uint64_t(__ballot(accept && lane < gamma));
    const int lead = rej == 0 ? kWave : __builtin_ctzll(rej);
    k = lead < gamma ? lead : gamma;
  } else if (lane < gamma) {
    if (out_p) out_p[b * gamma + lane] = NAN;
    if (out_q) out_q[b * gamma + lane] = NAN;
  }

  // Accepted prefix now; the drawn token at position k is written by the draw kernel.
  for (int i = lane; i <= gamma; i += kWave) {
    int32_t v = -1;
    if (i < k) v = x;  // i < k <= gamma <= 64 only on the first pass, where lane i holds x_i
    if (fallback && i == 0) v = 0;
    out_tokens[b * (gamma + 1) + i] = v;
  }
  if (lane == 0) {
    seq[b] = SeqDecision{k, fallback ? kDrawNone : (k < gamma ? kDrawResidual : kDrawBonus),
                         status, 0};
    if (fallback) {
      out_nacc[b] = 0;
      if (out_status) out_status[b] = status;
    }
  }
}

// ------------------------------------------------------------------------------------ 3. residual
template <typename T, int VW>
__global__ __launch_bounds__(kBlock) void k_chain_residual(
    const T* __restrict__ tgt, const T* __restrict__ drf, const float* __restrict__ temp,
    int gamma, int64_t V, int64_t nchunk, int64_t total, const RowPart* __restrict__ part,
    const RowStat* __restrict__ rowstat, const SeqDecision* __restrict__ seq,
    double* __restrict__ wres) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t w = int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x / kWave);
  if (w >= total) return;
  const int64_t b = w / nchunk;
  const int64_t c = w - b * nchunk;
  const SeqDecision d = seq[b];
  if (d.mode != kDrawResidual) return;
  const int R = 2 * gamma + 1;
  const int jt = d.k, jd = gamma + 1 + d.k;
  const RowPart pt = part[(b * R + jt) * nchunk + c];
  const RowPart pd = part[(b * R + jd) * nchunk + c];
  const float tb = temp[b];
  const float te = effective_temperature(tb);
  const double Td = te;
  const double A = chunk_scale(pt.m, rowstat[b * R + jt], Td);
  const double Bq = chunk_scale(pd.m, rowstat[b * R + jd], Td);
  const float k = log2e_over_t(te);

  float zt[kElemsPerLane], zd[kElemsPerLane];
  load_chunk<T, VW>(chain_row(tgt, drf, b, gamma, jt, V), V, c, lane, zt);
  load_chunk<T, VW>(chain_row(tgt, drf, b, gamma, jd, V), V, c, lane, zd);
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int i = 0; i < kElemsPerLane; ++i)
    acc[i & 3] += residual_term(zt[i], zd[i], pt.m, pd.m, k, A, Bq);
  const double s = wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
  if (lane == 0) wres[w] = s;
}

// ------------------------------------------------------------------------------------ 4. draw

// Running sum over the chunk masses of one sequence in chunk order.  Pass 1 returns the
// total; pass 2 (same association, hence the same bits) finds the first chunk whose
// inclusive sum exceeds tau and the exclusive sum before it.
template <typename MassFn>
__device__ double chunk_total(int64_t nchunk, int lane, MassFn mass) {
  double carry = 0.0;
  for (int64_t base = 0; base < nchunk; base += kWave) {
    const int64_t c = base + lane;
    const double v = c < nchunk ? mass(c) : 0.0;
    const double incl = wave_inclusive_scan(v, lane);
    carry += wave_broadcast(incl, kWave - 1);
  }
  return carry;
}

template <typename MassFn>
__device__ int64_t chunk_locate(int64_t nchunk, int lane, double tau, double* before,
                                MassFn mass) {
  double carry = 0.0;
  int64_t last_pos = -1;
  double last_before = 0.0;
  for (int64_t base = 0; base < nchunk; base += kWave) {
    const int64_t c = base + lane;
    const double v = c < nchunk ? mass(c) : 0.0;
    const double incl = wave_inclusive_scan(v, lane);
    const uint64_t hit = __ballot(c < nchunk && carry + incl > tau);
    if (hit) {
      const int L = __builtin_ctzll(hit);
      const double excl = wave_broadcast(incl - v, L);
      *before = carry + excl;
      return base + L;
    }
    const uint64_t pos = __ballot(c < nchunk && v > 0.0);
    if (pos) {
      const int L = 63 - __builtin_clzll(pos);
      last_before = carry + wave_broadcast(incl - v, L);
      last_pos = base + L;
    }
    carry += wave_broadcast(incl, kWave - 1);
  }
  // Not reached for tau < total; kept as a defined fallback (last chunk with mass).
  *before = last_before;
  return last_pos < 0 ? 0 : last_pos;
}

// Scan one chunk in token order and return the first element with positive weight at which
// the running weight exceeds tau_loc; if rounding leaves tau_loc unreached, the last element
// with positive weight.  A zero-weight element is never returned while the chunk holds weight.
template <int VW, typename TermFn>
__device__ int64_t chunk_scan(int64_t c, int64_t V, int lane, double tau_loc, TermFn term) {
  constexpr int NLD = kElemsPerLane / VW;
  double carry = 0.0;
  int last_pos = -1;
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    double w[VW];
    double ls = 0.0;
#pragma unroll
    for (int t = 0; t < VW; ++t) {
      w[t] = term(j * VW + t);
      ls += w[t];
    }
    const double incl = wave_inclusive_scan(ls, lane);
    double run = carry + (incl - ls);
    int cand = -1, lp = -1;
#pragma unroll
    for (int t = 0; t < VW; ++t) {
      run += w[t];
      if (w[t] > 0.0) {
        lp = chunk_offset<VW>(j, lane, t);
        if (cand < 0 && run > tau_loc) cand = lp;
      }
    }
    const uint64_t hit = __ballot(cand >= 0);
    if (hit) return c * kChunk + __shfl(cand, __builtin_ctzll(hit), kWave);
    last_pos = max(last_pos, wave_max_int(lp));
    carry += wave_broadcast(incl, kWave - 1);
  }
  const int64_t first = c * kChunk;
  if (last_pos >= 0) return first + last_pos;
  return first < V ? first : V - 1;
}

template <typename T, int VW>
__global__ __launch_bounds__(kWave) void k_chain_draw(
    const T* __restrict__ tgt, const T* __restrict__ drf, const float* __restrict__ uni,
    const float* __restrict__ temp, int gamma, int64_t V, int64_t nchunk,
    const RowPart* __restrict__ part, const RowStat* __restrict__ rowstat,
    const SeqDecision* __restrict__ seq, const double* __restrict__ wres,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_nacc,
    int32_t* __restrict__ out_status) {
  const int64_t b = blockIdx.x;
  const int lane = threadIdx.x;
  const SeqDecision d = seq[b];
  if (d.mode == kDrawNone) return;
  const int R = 2 * gamma + 1;
  const int k = d.k;
  int status = d.status;
  const float tb = temp[b];
  const float te = effective_temperature(tb);
  const double Td = te;
  const float kk = log2e_over_t(te);
  const double u = uni[b * (gamma + 1) + gamma];
  const double* wr = wres + b * nchunk;

  bool residual = d.mode == kDrawResidual;
  if (residual) {
    const double W = chunk_total(nchunk, lane, [&](int64_t c) { return wr[c]; });
    if (!(W > 0.0)) {
      residual = false;
      status |= SV_ROW_RESIDUAL_ZERO;
    }
  }

  int64_t y;
  if (residual) {
    auto mass = [&](int64_t c) { return wr[c]; };
    const double W = chunk_total(nchunk, lane, mass);
    double before = 0.0;
    const int64_t cs = chunk_locate(nchunk, lane, u * W, &before, mass);
    const int jt = k, jd = gamma + 1 + k;
    const RowPart pt = part[(b * R + jt) * nchunk + cs];
    const RowPart pd = part[(b * R + jd) * nchunk + cs];
    const double A = chunk_scale(pt.m, rowstat[b * R + jt], Td);
    const double Bq = chunk_scale(pd.m, rowstat[b * R + jd], Td);
    float zt[kElemsPerLane], zd[kElemsPerLane];
    load_chunk<T, VW>(chain_row(tgt, drf, b, gamma, jt, V), V, cs, lane, zt);
    load_chunk<T, VW>(chain_row(tgt, drf, b, gamma, jd, V), V, cs, lane, zd);
    y = chunk_scan<VW>(cs, V, lane, u * W - before, [&](int i) {
      return residual_term(zt[i], zd[i], pt.m, pd.m, kk, A, Bq);
    });
  } else {
    // Bonus draw from p_gamma, or the zero-residual fallback from p_k.
    const int jr = d.mode == kDrawBonus ? gamma : k;
    const RowStat srow = rowstat[b * R + jr];
    const RowPart* pp = part + (b * R + jr) * nchunk;
    auto mass = [&](int64_t c) {
      const RowPart q = pp[c];
      return q.s * chunk_scale(q.m, srow, Td);
    };
    const double W = chunk_total(nchunk, lane, mass);
    double before = 0.0;
    const double tau = u * W;
    const int64_t cs = chunk_locate(nchunk, lane, tau, &before, mass);
    const RowPart pc = pp[cs];
    const double scale = chunk_scale(pc.m, srow, Td);
    float z[kElemsPerLane];
    load_chunk<T, VW>(chain_row(tgt, drf, b, gamma, jr, V), V, cs, lane, z);
    const double tau_loc = scale > 0.0 ? (tau - before) / scale : 0.0;
    y = chunk_scan<VW>(cs, V, lane, tau_loc,
                       [&](int i) { return double(softmax_term(z[i], pc.m, kk)); });
  }
  if (lane == 0) {
    out_tokens[b * (gamma + 1) + k] = int32_t(y);
    out_nacc[b] = k;
    if (out_status) out_status[b] = status;
  }
}

template <typename T, int VW>
hipError_t run_chain(const ChainArgs& a, hipStream_t s) {
  const ChainLayout L = chain_layout(a.B, a.gamma, a.V);
  RowPart* part = reinterpret_cast<RowPart*>(a.ws + L.off_part);
  RowStat* rowstat = reinterpret_cast<RowStat*>(a.ws + L.off_rowstat);
  SeqDecision* seq = reinterpret_cast<SeqDecision*>(a.ws + L.off_seq);
  double* wres = reinterpret_cast<double*>(a.ws + L.off_wres);
  const T* tgt = static_cast<const T*>(a.target);
  const T* drf = static_cast<const T*>(a.draft);
  const int64_t rows = int64_t(a.B) * (2 * a.gamma + 1);
  const int64_t total = rows * L.nchunk;

  hipError_t e = launch_kernel("chain_rowstats", k_chain_rowstats<T, VW>,
                               dim3(unsigned((total + kWavesPerBlock - 1) / kWavesPerBlock)),
                               dim3(kBlock), s, tgt, drf, a.temperature, a.gamma, a.V, L.nchunk,
                               total, part);
  if (e != hipSuccess) return e;
  e = launch_kernel("chain_decide", k_chain_decide<T>, dim3(unsigned(a.B)), dim3(kBlock), s, tgt, drf,
                    a.draft_tokens, a.uniforms, a.temperature, a.gamma, a.V, L.nchunk,
                    (const RowPart*)part, rowstat, seq, a.out_tokens, a.out_num_accepted,
                    a.out_p, a.out_q, a.out_status);
  if (e != hipSuccess) return e;
  const int64_t rtotal = int64_t(a.B) * L.nchunk;
  e = launch_kernel("chain_residual", k_chain_residual<T, VW>,
                    dim3(unsigned((rtotal + kWavesPerBlock - 1) / kWavesPerBlock)),
                    dim3(kBlock), s, tgt, drf, a.temperature, a.gamma, a.V, L.nchunk, rtotal,
                    (const RowPart*)part, (const RowStat*)rowstat, (const SeqDecision*)seq,
                    wres);
  if (e != hipSuccess) return e;
  return launch_kernel("chain_draw", k_chain_draw<T, VW>, dim3(unsigned(a.B)), dim3(kWave), s, tgt, drf,
                       a.uniforms, a.temperature, a.gamma, a.V, L.nchunk, (const RowPart*)part,
                       (const RowStat*)rowstat, (const SeqDecision*)seq, (const double*)wres,
                       a.out_tokens, a.out_num_accepted, a.out_status);
}

}  // namespace

hipError_t launch_chain(const ChainArgs& a, hipStream_t s) {
  if (a.dtype == SV_F32) return a.vec ? run_chain<float, 4>(a, s) : run_chain<float, 1>(a, s);
  return a.vec ? run_chain<uint16_t, 8>(a, s) : run_chain<uint16_t, 1>(a, s);
}

}  // namespace sv
