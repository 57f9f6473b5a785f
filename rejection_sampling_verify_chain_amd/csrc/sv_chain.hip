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
// sv_verify_chain takes one of three paths, chosen by measured thresholds (choose_path), all
// with the same bits: a single launch with one workgroup per sequence (chain_fused, for small
// rows or 192..256 sequences), the sweep followed by one workgroup per sequence (chain_finish),
// or the four launches below.  sv_verify_chain_lazy takes the positions in order and reads no
// row after the cut (lazy_form): one launch per position across the chip (chain_stage), or one
// workgroup per sequence (chain_lazy).  All launches go on the caller's stream, with no host
// synchronisation.  The four launches of the split path:
//   sweep     the single HBM sweep over all B*(2*gamma+1)*V logits: each wave owns one chunk
//             (2048 elements) of one logit row and writes its chunk max m_c and
//             S_c = sum exp((z - m_c)/T) (fp32 terms, fp64 sum).
//   decide    one workgroup per sequence merges the partials into each row's max and
//             normaliser (fp64, one wave per row), evaluates p_i(x_i), q_i(x_i) in fp64 with
//             one lane per position, and takes the cut k = number of leading accepts with one
//             ballot.
//   residual  one wave per chunk of a rejecting sequence sums the residual max(0, p_k - q_k)
//             over that chunk of target row k and draft row k.
//   draw      one wave per sequence draws y by inverse CDF: a running sum over the chunk
//             masses (the residual masses, or the bonus row's p masses from the sweep) locates
//             the chunk holding u*W, and that chunk is rescanned in token order.
// Fusing the per-sequence tails into the streaming kernels (a last-workgroup finisher) was
// measured slower: the finisher's registers lower the streaming kernel's occupancy, its
// latency-bound work stretches under a saturated memory system, and it lands on whichever
// XCD lags.
//
// Further down, the per-position acceptance rates and the draft-side sampler reuse the sweep,
// the row merge and the draw.

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "sv_device.h"
#include "sv_internal.h"
#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kBlock = 1024;  // decide: one wave per row of a sequence
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kResidualBlock = 256;  // residual: one chunk per wave

struct ChainParams {
  const void* tgt;
  const void* drf;
  const int32_t* toks;
  const float* uni;
  const float* temp;
  int gamma;
  int tgt_rows;  // target rows per sequence the sweep covers: gamma + 1 (verify) or gamma

  int64_t V;
  int64_t nchunk;
  RowPart* part;
  RowStat* rowstat;
  SeqDecision* seq;
  double* wres;
  int32_t* out_tokens;
  int32_t* out_nacc;
  float* out_p;
  float* out_q;
  int32_t* out_status;
  // Staged early exit only: per sequence, "reached position j" flags [B][2] (slot j & 1), the
  // checks that need no logit row [B], and the drafted tokens' target and draft logits
  // [B][gamma][2].
  int32_t* alive = nullptr;
  int32_t* hstat = nullptr;
  float* lz = nullptr;
};

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

// Residual weights of one chunk, max(0, p(x) - q(x)) = A * max(0, e_t(x) - lambda * e_d(x)):
// e_t, e_d are the chunk-local softmax terms of target and draft row k, A = exp((m_t,c - M_t)/T)
// / S_t scales e_t to p, and lambda = B / A with B the draft's scale.  Per element this is one
// fp32 FMA (the product is exact inside it, so the difference rounds once) and a max; A is
// applied per chunk in fp64.  A = 0 (target chunk all -inf) gives no residual mass; B = 0
// (draft chunk all -inf) gives lambda = 0 and e_d is not formed.
struct ResidualScale {
  double A;
  float lambda;
  bool qlive;
};

__device__ __forceinline__ ResidualScale residual_scale(double A, double Bq) {
  if (!(A > 0.0)) return ResidualScale{0.0, 0.0f, false};
  return ResidualScale{A, float(fmin(Bq / A, 3.40282347e38)), Bq > 0.0};
}

__device__ __forceinline__ float residual_term(float zt, float zd, float mt, float md, float k,
                                               const ResidualScale& rs) {
  const float et = softmax_term(zt, mt, k);
  const float ed = rs.qlive ? softmax_term(zd, md, k) : 0.0f;
  return fmaxf(0.0f, fmaf(-rs.lambda, ed, et));
}

// ------------------------------------------------------------------------------------ sweep

// Sum of exp((z - m)/T) over a lane's elements: fp32 terms added in groups of four in fp32 (two
// roundings deep), the group sums accumulated in fp64.
template <typename TermFn>
__device__ __forceinline__ double lane_term_sum(TermFn term) {
  double acc[2] = {0.0, 0.0};
#pragma unroll
  for (int i = 0; i < kElemsPerLane; i += 4) {
    const float t = (term(i) + term(i + 1)) + (term(i + 2) + term(i + 3));
    acc[(i >> 2) & 1] += double(t);
  }
  return acc[0] + acc[1];
}

// One wave, one loaded chunk -> (chunk max, fp64 sum of exp((z - max)/T)).  Branch-free: a
// chunk with no value above -inf takes 0 as the exponent's reference, so its -inf terms are
// exp(-inf) = 0 and a NaN still poisons the sum (as does a +inf maximum, through inf - inf).
__device__ __forceinline__ RowPart reduce_chunk(const float (&z)[kElemsPerLane], float k) {
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kElemsPerLane; ++i) m = fmaxf(m, z[i]);
  m = wave_max(m);
  const float ref = m == -INFINITY ? 0.0f : m;
  const double s = wave_sum(lane_term_sum([&](int i) { return softmax_term(z[i], ref, k); }));
  return RowPart{m, 0, s};
}

// ------------------------------------------------------------------------------------ draw

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

// -------------------------------------------------------------------------------------- decide

// One wave merges the chunk partials of one row into (M, S, valid): M = max_c m_c and
// S = sum_c S_c exp((m_c - M)/T) in fp64.  Partials are fetched kMergeBatch per lane at a
// time, all loads in flight together; rows of up to 64 * kMergeBatch chunks are read once.

__device__ RowStat merge_row(const RowPart* pp, int64_t nchunk, int lane, double Td) {
  const bool single = nchunk <= int64_t(kWave) * kMergeBatch;
  RowPart r[kMergeBatch];
  float mloc = -INFINITY;
  for (int64_t base = 0; base < nchunk; base += int64_t(kWave) * kMergeBatch) {
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int64_t c = base + i * kWave + lane;
      r[i] = c < nchunk ? pp[c] : RowPart{-INFINITY, 0, 0.0};
    }
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) mloc = fmaxf(mloc, r[i].m);
  }
  const float m = wave_max(mloc);
  const bool finite_max = (m > -INFINITY) && (m < INFINITY);
  double s = 0.0;
  if (finite_max) {
    for (int64_t base = 0; base < nchunk; base += int64_t(kWave) * kMergeBatch) {
      if (!single) {
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) {
          const int64_t c = base + i * kWave + lane;
          r[i] = c < nchunk ? pp[c] : RowPart{-INFINITY, 0, 0.0};
        }
      }
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const double f = r[i].m == -INFINITY ? 0.0 : exp((double(r[i].m) - double(m)) / Td);
        s += r[i].s * f;  // a NaN partial survives the zero factor
      }
    }
  }
  s = wave_sum(s);
  return RowStat{m, finite_max && (s > 0.0) && (s < INFINITY), s};
}

struct DecideShared {
  RowStat st[2 * kMaxGamma + 1];
};

// The drafted token of position `lane` (lanes < gamma of one wave) and the target and draft
// logits it picks, fetched ahead of the decision.
struct Drafted {
  int x;
  bool bad;  // x outside [0, V)
  float zt, zd;
};

template <typename T>
__device__ __forceinline__ Drafted gather_drafted(const ChainParams& p, int64_t b, int lane) {
  Drafted g{0, false, 0.0f, 0.0f};
  if (lane < p.gamma) {
    const T* tgt = static_cast<const T*>(p.tgt);
    const T* drf = static_cast<const T*>(p.drf);
    g.x = p.toks[b * p.gamma + lane];
    g.bad = (g.x < 0) || (int64_t(g.x) >= p.V);
    if (!g.bad) {
      g.zt = widen(chain_row(tgt, drf, b, p.gamma, lane, p.V)[g.x]);
      g.zd = widen(chain_row(tgt, drf, b, p.gamma, p.gamma + 1 + lane, p.V)[g.x]);
    }
  }
  return g;
}

// The decision of sequence b from its row statistics st[0 .. 2*gamma] (one wave, lane i =
// position i): input checks, p_i(x_i) and q_i(x_i) in fp64, the accept bits and the cut.
// Writes p, q, the accepted prefix with its padding, and the fallback result; returns the
// decision (the same on every lane).
__device__ SeqDecision decide_from_stats(const ChainParams& p, int64_t b, const RowStat* st,
                                         const Drafted& g, float tb, double Td, int lane) {
  const int gamma = p.gamma;
  const int R = 2 * gamma + 1;
  int status = 0;
  if (!(tb > 0.0f && tb < INFINITY)) status |= SV_ROW_BAD_TEMPERATURE;
  bool bad = false;
  for (int i = lane; i <= gamma; i += kWave) {
    const float u = p.uni[b * (gamma + 1) + i];
    bad |= !(u >= 0.0f && u < 1.0f);
  }
  if (__any(bad)) status |= SV_ROW_BAD_UNIFORM;
  if (__any(g.bad)) status |= SV_ROW_TOKEN_RANGE;
  bad = false;
  for (int j = lane; j < R; j += kWave) bad |= !st[j].valid;
  if (__any(bad)) status |= SV_ROW_NONFINITE;

  const bool fallback = (status & (SV_ROW_TOKEN_RANGE | SV_ROW_NONFINITE |
                                   SV_ROW_BAD_TEMPERATURE | SV_ROW_BAD_UNIFORM)) != 0;
  int k = 0;
  if (!fallback) {
    bool accept = false;
    if (lane < gamma) {
      const RowStat a = st[lane];
      const RowStat d = st[gamma + 1 + lane];
      const double pi = exp((double(g.zt) - double(a.m)) / Td) / a.s;
      const double qi = exp((double(g.zd) - double(d.m)) / Td) / d.s;
      const double u = p.uni[b * (gamma + 1) + lane];
      if (qi > 0.0) {
        accept = u < fmin(1.0, pi / qi);
      } else {
        accept = (pi > 0.0) && (u < 1.0);  // ratio +inf; p = q = 0 rejects
      }
      if (p.out_p) p.out_p[b * gamma + lane] = float(pi);
      if (p.out_q) p.out_q[b * gamma + lane] = float(qi);
    }
    // k = number of leading ones of the accept mask.
    const uint64_t rej = ~uint64_t(__ballot(accept && lane < gamma));
    const int lead = rej == 0 ? kWave : __builtin_ctzll(rej);
    k = lead < gamma ? lead : gamma;
  } else if (lane < gamma) {
    if (p.out_p) p.out_p[b * gamma + lane] = NAN;
    if (p.out_q) p.out_q[b * gamma + lane] = NAN;
  }
  // Accepted prefix and padding; position k is written by the draw.
  for (int i = lane; i <= gamma; i += kWave) {
    int32_t v = -1;
    if (i < k) v = g.x;  // i < k <= gamma <= 64 only on the first pass, where lane i holds x_i
    if (fallback && i == 0) v = 0;
    p.out_tokens[b * (gamma + 1) + i] = v;
  }
  if (fallback && lane == 0) {
    p.out_nacc[b] = 0;
    if (p.out_status) p.out_status[b] = status;
  }
  return SeqDecision{k, fallback ? kDrawNone : (k < gamma ? kDrawResidual : kDrawBonus), status,
                     0};
}

// The decision for sequence b from the chunk partials of its rows (all threads of the
// sequence's workgroup).  Wave 0 first fetches the drafted tokens' logits, so that those
// dependent loads overlap the partials' merge.
template <typename T, int VW>
__device__ void decide_sequence(const ChainParams& p, int64_t b, DecideShared& sh) {
  const int R = 2 * p.gamma + 1;
  const int wave = wave_id();
  const int lane = threadIdx.x & (kWave - 1);
  const float tb = uniform_load(p.temp, b);
  const double Td = effective_temperature(tb);
  Drafted g{0, false, 0.0f, 0.0f};
  if (wave == 0) g = gather_drafted<T>(p, b, lane);

  // Row max and normaliser of every row of the sequence, one wave per row.
  for (int j = wave; j < R; j += kWavesPerBlock) {
    const RowStat st = merge_row(p.part + (b * R + j) * p.nchunk, p.nchunk, lane, Td);
    if (lane == 0) {
      sh.st[j] = st;
      p.rowstat[b * R + j] = st;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  const SeqDecision d = decide_from_stats(p, b, sh.st, g, tb, Td, lane);
  if (lane == 0) p.seq[b] = d;
}

// Inverse-CDF step over chunk masses (one wave): total W of the masses in chunk order, then
// the first chunk whose running sum exceeds u*W, and the running sum before it.  Lane l holds
// kLocateBatch consecutive chunks of a batch, so rows of up to 64 * kLocateBatch chunks load
// their masses once, all in flight together.  If rounding leaves u*W unreached, the last chunk
// with positive mass is returned.
constexpr int kLocateBatch = 4;

struct Located {
  int64_t chunk;
  double before;  // running sum of the masses of the chunks before it
  double total;
};

// One batch of the search: lane l holds the masses v of chunks base + l * kLocateBatch + i.
// Given the running sum `carry` of the earlier batches, finds the first chunk whose running sum
// exceeds tau (hit), and otherwise updates the last chunk with positive mass; returns the
// batch's total mass.
struct LocateState {
  int64_t last_c = -1;
  double last_before = 0.0;
  bool hit = false;
  Located at{0, 0.0, 0.0};
};

__device__ __forceinline__ double locate_batch(const double (&v)[kLocateBatch], int64_t base,
                                               int lane, double carry, double tau, double total,
                                               LocateState& ls_state) {
  constexpr int NB = kLocateBatch;
  double ls = 0.0;
#pragma unroll
  for (int i = 0; i < NB; ++i) ls += v[i];
  const double incl = wave_inclusive_scan(ls, lane);
  double run = carry + (incl - ls);
  int64_t cand = -1, lp = -1;
  double cand_before = 0.0, lp_before = 0.0;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int64_t c = base + int64_t(lane) * NB + i;
    const double prev = run;
    run += v[i];
    if (v[i] > 0.0) {
      lp = c;
      lp_before = prev;
      if (cand < 0 && run > tau) {
        cand = c;
        cand_before = prev;
      }
    }
  }
  const uint64_t hit = __ballot(cand >= 0);
  if (hit) {
    const int L = __builtin_ctzll(hit);
    ls_state.hit = true;
    ls_state.at = Located{__shfl(cand, L, kWave), wave_broadcast(cand_before, L), total};
  }
  const uint64_t pos = __ballot(lp >= 0);
  if (pos) {
    const int L = 63 - __builtin_clzll(pos);
    ls_state.last_c = __shfl(lp, L, kWave);
    ls_state.last_before = wave_broadcast(lp_before, L);
  }
  return wave_broadcast(incl, kWave - 1);
}

template <typename MassFn>
__device__ Located locate_chunk(int64_t nchunk, int lane, double u, MassFn mass) {
  constexpr int NB = kLocateBatch;
  const int64_t per = int64_t(kWave) * NB;
  const bool single = nchunk <= per;
  double v[NB];
  double carry = 0.0;
  for (int64_t base = 0; base < nchunk; base += per) {
    double ls = 0.0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t c = base + int64_t(lane) * NB + i;
      v[i] = c < nchunk ? mass(c) : 0.0;
      ls += v[i];
    }
    carry += wave_broadcast(wave_inclusive_scan(ls, lane), kWave - 1);
  }
  const double total = carry;
  const double tau = u * total;
  carry = 0.0;
  LocateState st;
  for (int64_t base = 0; base < nchunk; base += per) {
    if (!single) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int64_t c = base + int64_t(lane) * NB + i;
        v[i] = c < nchunk ? mass(c) : 0.0;
      }
    }
    carry += locate_batch(v, base, lane, carry, tau, total, st);
    if (st.hit) return st.at;
  }
  return Located{st.last_c < 0 ? 0 : st.last_c, st.last_before, total};
}

// The same search over a row of at most 64 * kLocateBatch chunks whose masses the lanes already
// hold: v[i] = mass of chunk lane * kLocateBatch + i (0 past the row).
__device__ Located locate_chunk_held(const double (&v)[kLocateBatch], int lane, double u) {
  double ls = 0.0;
#pragma unroll
  for (int i = 0; i < kLocateBatch; ++i) ls += v[i];
  const double total = wave_broadcast(wave_inclusive_scan(ls, lane), kWave - 1);
  LocateState st;
  locate_batch(v, 0, lane, 0.0, u * total, total, st);
  if (st.hit) return st.at;
  return Located{st.last_c < 0 ? 0 : st.last_c, st.last_before, total};
}

// Where the draw finds a sequence's row statistics, chunk partials and residual masses.
// WorkspaceSrc reads the workspace written by earlier kernels: wave-uniform records through the
// scalar cache (issued beside the vector loads they do not depend on), the per-lane chunk masses
// with vector loads.  LdsSrc reads the copies that the one-workgroup path keeps in LDS.
struct WorkspaceSrc {
  const ChainParams& p;
  int64_t b;
  __device__ RowStat stat(int j) const { return uniform_load(p.rowstat, b * (2 * p.gamma + 1) + j); }
  __device__ RowPart part(int j, int64_t c) const {
    return uniform_load(p.part, (b * (2 * p.gamma + 1) + j) * p.nchunk + c);
  }
  __device__ RowPart part_lane(int j, int64_t c) const {
    return p.part[(b * (2 * p.gamma + 1) + j) * p.nchunk + c];
  }
  __device__ double wres(int64_t c) const { return p.wres[b * p.nchunk + c]; }
};

struct LdsSrc {
  const RowStat* st;   // [2 * gamma + 1]
  const RowPart* prt;  // [2 * gamma + 1][nchunk]
  const double* wr;    // [nchunk]
  int64_t nchunk;
  __device__ RowStat stat(int j) const { return st[j]; }
  __device__ RowPart part(int j, int64_t c) const { return prt[j * nchunk + c]; }
  __device__ RowPart part_lane(int j, int64_t c) const { return prt[j * nchunk + c]; }
  __device__ double wres(int64_t c) const { return wr[c]; }
};

// Draw of sequence b (one wave): residual draw over the residual chunk masses (falling back to
// p_k if they sum to zero), or the bonus draw from p_gamma over the sweep's chunk masses.  It
// takes three dependent memory round trips: the decision, the chunk masses, the located chunk.
template <typename T, int VW, typename Src>
__device__ void draw_sequence(const ChainParams& p, int64_t b, const SeqDecision& d,
                              const Src& src) {
  const T* tgt = static_cast<const T*>(p.tgt);
  const T* drf = static_cast<const T*>(p.drf);
  const int gamma = p.gamma;
  const int64_t V = p.V, nchunk = p.nchunk;
  const int lane = threadIdx.x & (kWave - 1);
  const float te = effective_temperature(uniform_load(p.temp, b));
  const double Td = te;
  const float kk = log2e_over_t(te);
  const int k = d.k;
  int status = d.status;
  const double u = uniform_load(p.uni, b * (gamma + 1) + gamma);

  int64_t y = -1;
  if (d.mode == kDrawResidual) {
    const int jt = k, jd = gamma + 1 + k;
    const RowStat st_t = src.stat(jt);
    const RowStat st_d = src.stat(jd);
    const Located at = locate_chunk(nchunk, lane, u, [&](int64_t c) { return src.wres(c); });
    if (at.total > 0.0) {
      const int64_t cs = at.chunk;
      const int nvalid = chunk_valid(V, cs);
      RawChunk<T, VW> rt, rd;
      load_raw<T, VW>(chain_row(tgt, drf, b, gamma, jt, V) + cs * kChunk, nvalid, lane, rt);
      load_raw<T, VW>(chain_row(tgt, drf, b, gamma, jd, V) + cs * kChunk, nvalid, lane, rd);
      const RowPart pt = src.part(jt, cs);
      const RowPart pd = src.part(jd, cs);
      const ResidualScale rs =
          residual_scale(chunk_scale(pt.m, st_t, Td), chunk_scale(pd.m, st_d, Td));
      float zt[kElemsPerLane], zd[kElemsPerLane];
      unpack_chunk<T, VW>(rt, nvalid, lane, zt);
      unpack_chunk<T, VW>(rd, nvalid, lane, zd);
      const double tau_loc = rs.A > 0.0 ? (u * at.total - at.before) / rs.A : 0.0;
      y = chunk_scan<VW>(cs, V, lane, tau_loc, [&](int i) {
        return double(residual_term(zt[i], zd[i], pt.m, pd.m, kk, rs));
      });
    } else {
      status |= SV_ROW_RESIDUAL_ZERO;
    }
  }
  if (y < 0) {
    // Bonus draw from p_gamma, or the zero-residual fallback from p_k.
    const int jr = d.mode == kDrawBonus ? gamma : k;
    const RowStat srow = src.stat(jr);
    const Located at = locate_chunk(nchunk, lane, u, [&](int64_t c) {
      const RowPart q = src.part_lane(jr, c);
      return q.s * chunk_scale(q.m, srow, Td);
    });
    const int64_t cs = at.chunk;
    const int nvalid = chunk_valid(V, cs);
    RawChunk<T, VW> r;
    load_raw<T, VW>(chain_row(tgt, drf, b, gamma, jr, V) + cs * kChunk, nvalid, lane, r);
    const RowPart pc = src.part(jr, cs);
    const double scale = chunk_scale(pc.m, srow, Td);
    float z[kElemsPerLane];
    unpack_chunk<T, VW>(r, nvalid, lane, z);
    const double tau_loc = scale > 0.0 ? (u * at.total - at.before) / scale : 0.0;
    y = chunk_scan<VW>(cs, V, lane, tau_loc,
                       [&](int i) { return double(softmax_term(z[i], pc.m, kk)); });
  }
  if (lane == 0) {
    p.out_tokens[b * (gamma + 1) + k] = int32_t(y);
    p.out_nacc[b] = k;
    if (p.out_status) p.out_status[b] = status;
  }
}

// ------------------------------------------------------------------------------------ kernels

template <typename T, int VW>
__global__ __launch_bounds__(kStreamBlock<T>, kStreamWavesPerSimd<VW>) void k_chain_sweep(
    ChainParams p, int64_t total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = int64_t(blockIdx.x) * (kStreamBlock<T> / kWave) + wave_id();
  const T* tgt = static_cast<const T*>(p.tgt);
  const T* drf = static_cast<const T*>(p.drf);
  // Row j of sequence b: target row j for j < tgt_rows, else draft row j - tgt_rows.
  stream_wave<RawChunk<T, VW>, kUnitsPerWave<T>>(
      gw, total, p.nchunk, p.tgt_rows + p.gamma,
      [&](const Unit& k, RawChunk<T, VW>& r) {
        const T* row = k.j < p.tgt_rows ? tgt + (k.b * (p.gamma + 1) + k.j) * p.V
                                        : drf + (k.b * p.gamma + (k.j - p.tgt_rows)) * p.V;
        load_raw<T, VW>(row + int64_t(k.c) * kChunk, chunk_valid(p.V, k.c), lane, r);
      },
      [&](const Unit& k, const RawChunk<T, VW>& r) {
        float z[kElemsPerLane];
        unpack_chunk<T, VW>(r, chunk_valid(p.V, k.c), lane, z);
        const RowPart rp =
            reduce_chunk(z, log2e_over_t(effective_temperature(uniform_load(p.temp, k.b))));
        if (lane == 0) p.part[k.w] = rp;
      });
}

template <typename T, int VW>
__global__ __launch_bounds__(kBlock) void k_chain_decide(ChainParams p) {
  __shared__ DecideShared sh;
  decide_sequence<T, VW>(p, blockIdx.x, sh);
}

// Residual mass W_c of one chunk (one wave) from its loaded target and draft chunks, their chunk
// partials and the rows' statistics.  A chunk whose target part is all -inf (A = 0) has none.
template <typename T, int VW>
__device__ __forceinline__ double residual_chunk_mass(const RawChunk<T, VW>& rt,
                                                      const RawChunk<T, VW>& rd, int nvalid,
                                                      int lane, const RowPart& pt,
                                                      const RowPart& pd, const RowStat& st_t,
                                                      const RowStat& st_d, double Td, float kk) {
  const ResidualScale rs = residual_scale(chunk_scale(pt.m, st_t, Td), chunk_scale(pd.m, st_d, Td));
  float zt[kElemsPerLane], zd[kElemsPerLane];
  unpack_chunk<T, VW>(rt, nvalid, lane, zt);
  unpack_chunk<T, VW>(rd, nvalid, lane, zd);
  const double wsum = wave_sum(lane_term_sum(
      [&](int i) { return residual_term(zt[i], zd[i], pt.m, pd.m, kk, rs); }));
  return rs.A > 0.0 ? rs.A * wsum : 0.0;
}

// The wave's chunk loads of both rows are issued as soon as the decision (which row) is known;
// the chunk partials and row statistics that scale them arrive through the scalar cache while
// the chunk is in flight.  A chunk whose target part is all -inf (A = 0) is loaded too and adds
// nothing.
template <typename T, int VW>
__global__ __launch_bounds__(kResidualBlock) void k_chain_residual(ChainParams p, int64_t total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t w = int64_t(blockIdx.x) * (kResidualBlock / kWave) + wave_id();
  if (w >= total) return;  // wave-uniform
  const int64_t b = w / p.nchunk;
  const int64_t c = w - b * p.nchunk;
  const SeqDecision d = uniform_load(p.seq, b);
  if (d.mode != kDrawResidual) return;
  const int R = 2 * p.gamma + 1;
  const int jt = d.k, jd = p.gamma + 1 + d.k;
  const T* tgt = static_cast<const T*>(p.tgt);
  const T* drf = static_cast<const T*>(p.drf);
  const int nvalid = chunk_valid(p.V, c);
  RawChunk<T, VW> rt, rd;
  load_raw<T, VW>(chain_row(tgt, drf, b, p.gamma, jt, p.V) + c * kChunk, nvalid, lane, rt);
  load_raw<T, VW>(chain_row(tgt, drf, b, p.gamma, jd, p.V) + c * kChunk, nvalid, lane, rd);
  const float te = effective_temperature(uniform_load(p.temp, b));
  const double w_c = residual_chunk_mass<T, VW>(
      rt, rd, nvalid, lane, uniform_load(p.part, (b * R + jt) * p.nchunk + c),
      uniform_load(p.part, (b * R + jd) * p.nchunk + c), uniform_load(p.rowstat, b * R + jt),
      uniform_load(p.rowstat, b * R + jd), double(te), log2e_over_t(te));
  if (lane == 0) p.wres[w] = w_c;
}

template <typename T, int VW>
__global__ __launch_bounds__(kWave) void k_chain_draw(ChainParams p) {
  const int64_t b = blockIdx.x;
  const SeqDecision d = uniform_load(p.seq, b);
  if (d.mode == kDrawNone) return;  // fallback: the decide kernel wrote the result
  draw_sequence<T, VW>(p, b, d, WorkspaceSrc{p, b});
}

// ------------------------------------------------------------------------ one workgroup per sequence
//
// Sequences with small rows run every step in a single launch: one workgroup per sequence sweeps
// its 2*gamma+1 rows (a chunk per wave at a time), keeps the chunk partials, row statistics,
// decision and residual masses in LDS, and separates the steps with workgroup barriers.  Each
// step calls the same device functions as the multi-kernel path, so both give the same bits.
// With SWEPT the rows were swept by chain_sweep across the whole chip, and the workgroup copies
// the sequence's chunk partials into LDS instead (chain_finish: the sweep plus one launch for
// the decide, residual and draw steps); it also stores the row statistics in the workspace.
constexpr int kFusedBlock = 1024;
constexpr int kFusedWaves = kFusedBlock / kWave;
template <typename T>
constexpr int kFusedUnits = kUnitsPerWave<T>;  // chunks per wave in flight

struct FusedShared {
  RowStat st[2 * kMaxGamma + 1];
  SeqDecision d;
};

// The body of chain_fused and chain_finish (all threads of the sequence's workgroup); fused_lds
// is the launch's dynamic LDS: partials [R][nchunk], then residual masses [nchunk].
template <typename T, int VW, bool SWEPT>
__device__ __forceinline__ void one_workgroup_chain(const ChainParams& p, unsigned char* fused_lds,
                                                    FusedShared& sh) {
  const int64_t b = blockIdx.x;
  const int gamma = p.gamma;
  const int R = 2 * gamma + 1;
  const int64_t V = p.V, nchunk = p.nchunk;
  const int wave = wave_id();
  const int lane = threadIdx.x & (kWave - 1);
  RowPart* prt = reinterpret_cast<RowPart*>(fused_lds);
  double* wr = reinterpret_cast<double*>(fused_lds + sizeof(RowPart) * size_t(R) * size_t(nchunk));
  const T* tgt = static_cast<const T*>(p.tgt);
  const T* drf = static_cast<const T*>(p.drf);
  const float tb = uniform_load(p.temp, b);
  const float te = effective_temperature(tb);
  const double Td = te;
  const float kk = log2e_over_t(te);

  Drafted g{0, false, 0.0f, 0.0f};
  if (wave == 0) g = gather_drafted<T>(p, b, lane);

  const int units = R * int(nchunk);  // fits in int: the LDS budget bounds it
  if constexpr (SWEPT) {
    const RowPart* part = p.part + b * int64_t(units);
    for (int w = int(threadIdx.x); w < units; w += kFusedBlock) prt[w] = part[w];
  } else {
  // Sweep: the chunk partials of every row (virtual row j as in chain_row), kFusedUnits
  // consecutive units per wave with all their loads in flight (two fp32 chunks per wave spill at
  // the 128 registers a 1024-thread workgroup allows); a unit past the end reloads the last one
  // and is not reduced.
  constexpr int U = kFusedUnits<T>;
  for (int w0 = wave * U; w0 < units; w0 += kFusedWaves * U) {
    RawChunk<T, VW> r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = min(w0 + u, units - 1);
      const int j = w / int(nchunk);
      const int c = w - j * int(nchunk);
      load_raw<T, VW>(chain_row(tgt, drf, b, gamma, j, V) + int64_t(c) * kChunk,
                      chunk_valid(V, c), lane, r[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = w0 + u;
      if (w < units) {  // wave-uniform
        const int c = w - (w / int(nchunk)) * int(nchunk);
        float z[kElemsPerLane];
        unpack_chunk<T, VW>(r[u], chunk_valid(V, c), lane, z);
        const RowPart rp = reduce_chunk(z, kk);
        if (lane == 0) prt[w] = rp;
      }
    }
  }
  }
  __syncthreads();
  for (int j = wave; j < R; j += kFusedWaves) {
    const RowStat st = merge_row(prt + int64_t(j) * nchunk, nchunk, lane, Td);
    if (lane == 0) {
      sh.st[j] = st;
      if (SWEPT) p.rowstat[b * R + j] = st;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const SeqDecision d = decide_from_stats(p, b, sh.st, g, tb, Td, lane);
    if (lane == 0) sh.d = d;
  }
  __syncthreads();
  const SeqDecision d = sh.d;
  if (d.mode == kDrawNone) return;  // the whole workgroup: the decision wrote the result
  if (d.mode == kDrawResidual) {     // the whole workgroup
    const int jt = d.k, jd = gamma + 1 + d.k;
    for (int64_t c = wave; c < nchunk; c += kFusedWaves) {
      const int nvalid = chunk_valid(V, c);
      RawChunk<T, VW> rt, rd;
      load_raw<T, VW>(chain_row(tgt, drf, b, gamma, jt, V) + c * kChunk, nvalid, lane, rt);
      load_raw<T, VW>(chain_row(tgt, drf, b, gamma, jd, V) + c * kChunk, nvalid, lane, rd);
      const double w_c = residual_chunk_mass<T, VW>(rt, rd, nvalid, lane, prt[jt * nchunk + c],
                                                    prt[jd * nchunk + c], sh.st[jt], sh.st[jd],
                                                    Td, kk);
      if (lane == 0) wr[c] = w_c;
    }
    __syncthreads();
  }
  if (wave != 0) return;
  draw_sequence<T, VW>(p, b, d, LdsSrc{sh.st, prt, wr, nchunk});
}

template <typename T, int VW>
__global__ __launch_bounds__(kFusedBlock) void k_chain_fused(ChainParams p) {
  extern __shared__ __align__(16) unsigned char fused_lds[];
  __shared__ FusedShared sh;
  one_workgroup_chain<T, VW, false>(p, fused_lds, sh);
}

template <typename T, int VW>
__global__ __launch_bounds__(kFusedBlock) void k_chain_finish(ChainParams p) {
  extern __shared__ __align__(16) unsigned char fused_lds[];
  __shared__ FusedShared sh;
  one_workgroup_chain<T, VW, true>(p, fused_lds, sh);
}

// ------------------------------------------------------------------------ early exit (positions in order)
//
// One workgroup per sequence takes the positions in order: it sweeps target row i and draft row
// i into LDS, merges them, and tests position i; it stops at the first rejection (residual
// masses over the same two rows, then the draw) or, after gamma accepts, sweeps target row gamma
// for the bonus draw.  Rows after the cut are never read.  Each step calls the same device
// functions as the other paths, so for inputs whose rows are all finite the outputs are theirs
// bit for bit; only non-finite values in unread rows go unseen.

// Chunks per wave in flight when one workgroup sweeps a row pair: 8 KiB of logits (two bf16
// chunks measured 2-3% faster here than one, unlike the chip-wide sweeps).
template <typename T>
constexpr int kLazyUnits = 4 / int(sizeof(T));

// The draw's records for the row pair in LDS: slot 0 holds target row j <= gamma, slot 1 draft row
// j > gamma.
struct PairSrc {
  const RowStat* st2;  // [2]
  const RowPart* prt;  // [2][nchunk]
  const double* wr;    // [nchunk]
  int64_t nchunk;
  int gamma;
  __device__ int slot(int j) const { return j > gamma ? 1 : 0; }
  __device__ RowStat stat(int j) const { return st2[slot(j)]; }
  __device__ RowPart part(int j, int64_t c) const { return prt[slot(j) * nchunk + c]; }
  __device__ RowPart part_lane(int j, int64_t c) const { return prt[slot(j) * nchunk + c]; }
  __device__ double wres(int64_t c) const { return wr[c]; }
};

struct LazyShared {
  RowStat st2[2];
  int32_t state;  // after a position's test: 0 accepted, 1 rejected, 2 non-finite row
  int32_t status;
};

// Chunk partials of rows j0 (slot 0) and, if nrows == 2, j1 (slot 1) into prt (all threads).
template <typename T, int VW>
__device__ __forceinline__ void sweep_pair(const ChainParams& p, int64_t b, int j0, int j1,
                                           int nrows, RowPart* prt, float kk, int wave, int lane) {
  const T* tgt = static_cast<const T*>(p.tgt);
  const T* drf = static_cast<const T*>(p.drf);
  const int nchunk = int(p.nchunk);
  constexpr int U = kLazyUnits<T>;
  const int units = nrows * nchunk;
  for (int w0 = wave * U; w0 < units; w0 += kFusedWaves * U) {
    RawChunk<T, VW> r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = min(w0 + u, units - 1);
      const int slot = w / nchunk;
      const int c = w - slot * nchunk;
      load_raw<T, VW>(chain_row(tgt, drf, b, p.gamma, slot ? j1 : j0, p.V) + int64_t(c) * kChunk,
                      chunk_valid(p.V, c), lane, r[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = w0 + u;
      if (w < units) {  // wave-uniform
        const int c = w - (w / nchunk) * nchunk;
        float z[kElemsPerLane];
        unpack_chunk<T, VW>(r[u], chunk_valid(p.V, c), lane, z);
        const RowPart rp = reduce_chunk(z, kk);
        if (lane == 0) prt[w] = rp;
      }
    }
  }
}

// The fallback result of sequence b (one wave): k = 0, tokens [0, -1, ...], p and q NaN.
__device__ __forceinline__ void write_fallback(const ChainParams& p, int64_t b, int status,
                                               int lane) {
  for (int i = lane; i <= p.gamma; i += kWave) p.out_tokens[b * (p.gamma + 1) + i] = i == 0 ? 0 : -1;
  for (int i = lane; i < p.gamma; i += kWave) {
    if (p.out_p) p.out_p[b * p.gamma + i] = NAN;
    if (p.out_q) p.out_q[b * p.gamma + i] = NAN;
  }
  if (lane == 0) {
    p.out_nacc[b] = 0;
    if (p.out_status) p.out_status[b] = status;
  }
}

template <typename T, int VW>
__global__ __launch_bounds__(kFusedBlock) void k_chain_lazy(ChainParams p) {
  extern __shared__ __align__(16) unsigned char lazy_lds[];  // partials [2][nchunk], masses [nchunk]
  __shared__ LazyShared sh;
  const int64_t b = blockIdx.x;
  const int gamma = p.gamma;
  const int64_t V = p.V, nchunk = p.nchunk;
  const int wave = wave_id();
  const int lane = threadIdx.x & (kWave - 1);
  RowPart* prt = reinterpret_cast<RowPart*>(lazy_lds);
  double* wr = reinterpret_cast<double*>(lazy_lds + sizeof(RowPart) * 2 * size_t(nchunk));
  const T* tgt = static_cast<const T*>(p.tgt);
  const T* drf = static_cast<const T*>(p.drf);
  const float tb = uniform_load(p.temp, b);
  const float te = effective_temperature(tb);
  const double Td = te;
  const float kk = log2e_over_t(te);

  // Checks that read no logit row: temperature, uniforms, draft tokens.
  Drafted g{0, false, 0.0f, 0.0f};
  if (wave == 0) {
    g = gather_drafted<T>(p, b, lane);
    int status = 0;
    if (!(tb > 0.0f && tb < INFINITY)) status |= SV_ROW_BAD_TEMPERATURE;
    bool bad = false;
    for (int i = lane; i <= gamma; i += kWave) {
      const float u = p.uni[b * (gamma + 1) + i];
      bad |= !(u >= 0.0f && u < 1.0f);
    }
    if (__any(bad)) status |= SV_ROW_BAD_UNIFORM;
    if (__any(g.bad)) status |= SV_ROW_TOKEN_RANGE;
    if (lane == 0) sh.status = status;
  }
  __syncthreads();
  if (sh.status != 0) {  // the whole workgroup
    if (wave == 0) write_fallback(p, b, sh.status, lane);
    return;
  }

  int k = gamma;
  for (int i = 0; i < gamma; ++i) {
    sweep_pair<T, VW>(p, b, i, gamma + 1 + i, 2, prt, kk, wave, lane);
    __syncthreads();
    if (wave < 2) {
      const RowStat st = merge_row(prt + wave * nchunk, nchunk, lane, Td);
      if (lane == 0) sh.st2[wave] = st;
    }
    __syncthreads();
    if (wave == 0) {
      const RowStat a = sh.st2[0], d = sh.st2[1];
      int state = 2;
      if (a.valid && d.valid) {
        // Position i's test, on the logits lane i gathered (the eager path's arithmetic).
        const double zt = __shfl(g.zt, i, kWave), zd = __shfl(g.zd, i, kWave);
        const double pi = exp((zt - double(a.m)) / Td) / a.s;
        const double qi = exp((zd - double(d.m)) / Td) / d.s;
        const double u = p.uni[b * (gamma + 1) + i];
        const bool accept = qi > 0.0 ? u < fmin(1.0, pi / qi) : (pi > 0.0) && (u < 1.0);
        if (lane == 0) {
          if (p.out_p) p.out_p[b * gamma + i] = float(pi);
          if (p.out_q) p.out_q[b * gamma + i] = float(qi);
        }
        state = accept ? 0 : 1;
      }
      if (lane == 0) sh.state = state;
    }
    __syncthreads();
    const int state = sh.state;
    if (state == 2) {
      if (wave == 0) write_fallback(p, b, SV_ROW_NONFINITE, lane);
      return;
    }
    if (state == 1) {
      k = i;
      break;
    }
  }

  SeqDecision dec;
  if (k < gamma) {
    // Residual masses over the two rows still in LDS.
    const int jt = k, jd = gamma + 1 + k;
    for (int64_t c = wave; c < nchunk; c += kFusedWaves) {
      const int nvalid = chunk_valid(V, c);
      RawChunk<T, VW> rt, rd;
      load_raw<T, VW>(chain_row(tgt, drf, b, gamma, jt, V) + c * kChunk, nvalid, lane, rt);
      load_raw<T, VW>(chain_row(tgt, drf, b, gamma, jd, V) + c * kChunk, nvalid, lane, rd);
      const double w_c = residual_chunk_mass<T, VW>(rt, rd, nvalid, lane, prt[c],
                                                    prt[nchunk + c], sh.st2[0], sh.st2[1], Td, kk);
      if (lane == 0) wr[c] = w_c;
    }
    __syncthreads();
    dec = SeqDecision{k, kDrawResidual, 0, 0};
  } else {
    sweep_pair<T, VW>(p, b, gamma, gamma, 1, prt, kk, wave, lane);
    __syncthreads();
    if (wave == 0) {
      const RowStat st = merge_row(prt, nchunk, lane, Td);
      if (lane == 0) sh.st2[0] = st;
    }
    __syncthreads();
    if (!sh.st2[0].valid) {
      if (wave == 0) write_fallback(p, b, SV_ROW_NONFINITE, lane);
      return;
    }
    dec = SeqDecision{gamma, kDrawBonus, 0, 0};
  }
  if (wave != 0) return;
  // The accepted prefix, padding, and positions after the cut (never evaluated: p, q NaN).
  for (int i = lane; i <= gamma; i += kWave)
    if (i != k) p.out_tokens[b * (gamma + 1) + i] = i < k ? g.x : -1;
  for (int i = lane; i < gamma; i += kWave) {
    if (i > k && p.out_p) p.out_p[b * gamma + i] = NAN;
    if (i > k && p.out_q) p.out_q[b * gamma + i] = NAN;
  }
  draw_sequence<T, VW>(p, b, dec, PairSrc{sh.st2, prt, wr, nchunk, gamma});
}

// ------------------------------------------------------------------------ early exit, staged
//
// The positions in order with the whole chip on each: launch j (0 <= j <= gamma + 1) works on
// every sequence that reached position j - 1, in workgroups that each take a slice of its
// chunks.  Every workgroup first decides position j - 1 itself (waves 0 and 1 merge the chunk
// partials of target and draft row j - 1; at j = gamma + 1 only target row gamma, the bonus
// row), and workgroup 0 writes the sequence's outputs and, at a cut or the bonus row, the
// decision and row statistics.  After an accept the workgroup sweeps its slice of row pair j
// (target row gamma alone at j = gamma) into chunk partials and fetches the drafted token's two
// logits at position j; otherwise it exits.  Launch 0 sweeps pair 0 of every sequence and checks
// the inputs that need no logit row.  The multi-kernel path's residual and draw kernels then
// finish every sequence from the decisions.  Rows after the cut are never read, and each step
// calls the eager path's device functions on the same values, so the outputs agree with
// sv_verify_chain bit for bit (p and q after the cut excepted).

enum StageRole : int32_t { kStageExit = 0, kStageSweep = 1 };

constexpr int kStageBlock = 256;
constexpr int kStageWavesPerSimd = 8;
template <typename T>
constexpr int kStageUnits = (kStageBlock / kWave) * kUnitsPerWave<T>;  // chunks per workgroup

// Workgroups per sequence in launch j: enough for the largest slice work of that launch.
inline int stage_groups(int j, int gamma, int64_t nchunk, int units_per_group) {
  if (j > gamma) return 1;
  const int64_t units = (j < gamma ? 2 : 1) * nchunk;
  return int((units + units_per_group - 1) / units_per_group);
}

template <typename T, int VW>
__global__ __launch_bounds__(kStageBlock, kStageWavesPerSimd) void k_chain_stage(
    ChainParams p, int j, int G) {
  __shared__ RowStat st2[2];
  __shared__ int32_t role;
  const int64_t b = blockIdx.x / G;
  const int g = int(blockIdx.x - b * G);
  const bool lead = g == 0;  // writes the sequence's outputs
  const int gamma = p.gamma;
  const int R = 2 * gamma + 1;
  const int64_t nchunk = p.nchunk;
  const int wave = wave_id();
  const int lane = threadIdx.x & (kWave - 1);
  const T* tgt = static_cast<const T*>(p.tgt);
  const T* drf = static_cast<const T*>(p.drf);
  const float tb = uniform_load(p.temp, b);
  const float te = effective_temperature(tb);
  const double Td = te;
  const float kk = log2e_over_t(te);

  int r = kStageSweep;
  if (j == 0) {
    if (lead && wave == 0) {
      // Checks that read no logit row; launch 1 takes the fallback on them.
      int status = 0;
      if (!(tb > 0.0f && tb < INFINITY)) status |= SV_ROW_BAD_TEMPERATURE;
      bool bad = false;
      for (int i = lane; i <= gamma; i += kWave) {
        const float u = p.uni[b * (gamma + 1) + i];
        bad |= !(u >= 0.0f && u < 1.0f);
      }
      if (__any(bad)) status |= SV_ROW_BAD_UNIFORM;
      bad = false;
      for (int i = lane; i < gamma; i += kWave) {
        const int x = p.toks[b * gamma + i];
        bad |= (x < 0) || (int64_t(x) >= p.V);
      }
      if (__any(bad)) status |= SV_ROW_TOKEN_RANGE;
      if (lane == 0) {
        p.hstat[b] = status;
        p.alive[b * 2] = 1;
      }
    }
  } else {
    const int i = j - 1;  // the position decided here; i == gamma: the bonus row
    if (!uniform_load(p.alive, b * 2 + (i & 1))) {
      if (lead && threadIdx.x == 0) p.alive[b * 2 + (j & 1)] = 0;
      return;  // the whole workgroup: the flag is uniform
    }
    if (wave < (i < gamma ? 2 : 1)) {
      const RowStat st = merge_row(p.part + (b * R + (wave == 0 ? i : gamma + 1 + i)) * nchunk,
                                   nchunk, lane, Td);
      if (lane == 0) st2[wave] = st;
    }
    __syncthreads();
    if (wave == 0) {
      const RowStat a = st2[0];
      const RowStat d = i < gamma ? st2[1] : a;
      int status = i == 0 ? uniform_load(p.hstat, b) : 0;
      if (!a.valid || !d.valid) status |= SV_ROW_NONFINITE;
      int rr = kStageExit;
      if (status != 0) {
        if (lead) {
          write_fallback(p, b, status, lane);
          if (lane == 0) p.seq[b] = SeqDecision{0, kDrawNone, status, 0};
        }
      } else if (i == gamma) {
        if (lead && lane == 0) {
          p.rowstat[b * R + gamma] = a;
          p.seq[b] = SeqDecision{gamma, kDrawBonus, 0, 0};
        }
      } else {
        // Position i's test on the logits launch i fetched (the eager path's arithmetic).
        const int x = uniform_load(p.toks, b * gamma + i);
        const float zt = uniform_load(p.lz, (b * gamma + i) * 2);
        const float zd = uniform_load(p.lz, (b * gamma + i) * 2 + 1);
        const double pi = exp((double(zt) - double(a.m)) / Td) / a.s;
        const double qi = exp((double(zd) - double(d.m)) / Td) / d.s;
        const double u = uniform_load(p.uni, b * (gamma + 1) + i);
        const bool accept = qi > 0.0 ? u < fmin(1.0, pi / qi) : (pi > 0.0) && (u < 1.0);
        if (lead) {
          if (lane == 0) {
            if (p.out_p) p.out_p[b * gamma + i] = float(pi);
            if (p.out_q) p.out_q[b * gamma + i] = float(qi);
          }
          if (accept) {
            if (lane == 0) p.out_tokens[b * (gamma + 1) + i] = x;
          } else {
            // The cut: padding, and positions never evaluated (p, q NaN).
            for (int t = i + 1 + lane; t <= gamma; t += kWave) {
              p.out_tokens[b * (gamma + 1) + t] = -1;
              if (t < gamma && p.out_p) p.out_p[b * gamma + t] = NAN;
              if (t < gamma && p.out_q) p.out_q[b * gamma + t] = NAN;
            }
            if (lane == 0) {
              p.rowstat[b * R + i] = a;
              p.rowstat[b * R + gamma + 1 + i] = d;
              p.seq[b] = SeqDecision{i, kDrawResidual, 0, 0};
            }
          }
        }
        rr = accept ? kStageSweep : kStageExit;
      }
      if (lead && lane == 0) p.alive[b * 2 + (j & 1)] = rr == kStageSweep ? 1 : 0;
      if (lane == 0) role = rr;
    }
    __syncthreads();
    r = role;
  }

  constexpr int U = kUnitsPerWave<T>;
  const int64_t u0 = int64_t(g) * kStageUnits<T> + int64_t(wave) * U;
  if (r == kStageSweep) {
    if (lead && wave == 0 && j < gamma) {
      // The drafted token's logits at position j, for launch j + 1's test.
      const int x = uniform_load(p.toks, b * gamma + j);
      if (lane == 0 && x >= 0 && int64_t(x) < p.V) {
        p.lz[(b * gamma + j) * 2] = widen(chain_row(tgt, drf, b, gamma, j, p.V)[x]);
        p.lz[(b * gamma + j) * 2 + 1] = widen(chain_row(tgt, drf, b, gamma, gamma + 1 + j, p.V)[x]);
      }
    }
    const int64_t units = (j < gamma ? 2 : 1) * nchunk;
    RawChunk<T, VW> raw[U];
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int64_t w = min(u0 + t, units - 1);
      const int row = w < nchunk ? j : gamma + 1 + j;
      const int64_t c = w < nchunk ? w : w - nchunk;
      load_raw<T, VW>(chain_row(tgt, drf, b, gamma, row, p.V) + c * kChunk, chunk_valid(p.V, c),
                      lane, raw[t]);
    }
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int64_t w = u0 + t;
      if (w < units) {  // wave-uniform
        const int row = w < nchunk ? j : gamma + 1 + j;
        const int64_t c = w < nchunk ? w : w - nchunk;
        float z[kElemsPerLane];
        unpack_chunk<T, VW>(raw[t], chunk_valid(p.V, c), lane, z);
        const RowPart rp = reduce_chunk(z, kk);
        if (lane == 0) p.part[(b * R + row) * nchunk + c] = rp;
      }
    }
  }
}

// ------------------------------------------------------------------------------------ alpha

// Acceptance rate alpha_i = sum_x min(p_i(x), q_i(x)) of position i of sequence b (the Step 3
// accept probability averaged over x ~ q_i).  They follow a sweep whose partials hold, per
// sequence, tgt_rows target rows then gamma draft rows: target row i is partial row
// b * (tgt_rows + gamma) + i and draft row i is that plus tgt_rows (tgt_rows = gamma for the
// standalone acceptance rates, gamma + 1 when they follow chain verification, whose decide
// kernel has already merged the rows).  Kernels:
//   merge    one wave per row merges its chunk partials into (M, S) (standalone only).
//   overlap  one wave per (b, i, chunk c) adds s * sum_x min(ra e_t(x), rb e_d(x)) over chunk c
//            of target row i and draft row i, where e_t, e_d are the chunk-local softmax terms,
//            A and B the chunk scales taking them to p and q, s = max(A, B) and
//            (ra, rb) = (A, B) / s (one of them is 1, the other at most 1, so nothing
//            overflows).  A chunk where A or B is 0 adds nothing.  The chunk loads go out first;
//            the row statistics and chunk partials arrive through the scalar cache meanwhile.
//            Workgroups are sized like the sweep's (measured: 1024 threads for fp32, 256 for
//            bf16; a workgroup per (b, i) with waves looping over the chunks ran at 0.47 of
//            the HBM peak on 131 MB of bf16, this form at 0.68).
//   reduce   one wave per (b, i) adds the chunk sums in a fixed order (deterministic).
constexpr int kAlphaBlock = 256;

__device__ __forceinline__ int64_t alpha_target_row(const ChainParams& p, int64_t b, int i) {
  return b * (p.tgt_rows + p.gamma) + i;
}

__global__ __launch_bounds__(kAlphaBlock) void k_chain_alpha_merge(ChainParams p, int64_t rows) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = int64_t(blockIdx.x) * (kAlphaBlock / kWave) + wave_id();
  if (r >= rows) return;  // wave-uniform
  const int64_t b = r / (p.tgt_rows + p.gamma);
  const double Td = effective_temperature(uniform_load(p.temp, b));
  const RowStat st = merge_row(p.part + r * p.nchunk, p.nchunk, lane, Td);
  if (lane == 0) p.rowstat[r] = st;
}

template <typename T, int VW>
__global__ __launch_bounds__(kStreamBlock<T>) void k_chain_alpha(ChainParams p, double* chunk_sum,
                                                                int64_t total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t w = int64_t(blockIdx.x) * (kStreamBlock<T> / kWave) + wave_id();
  if (w >= total) return;  // wave-uniform
  const int gamma = p.gamma;
  const int64_t V = p.V, nchunk = p.nchunk;
  const int64_t pair = w / nchunk;
  const int64_t c = w - pair * nchunk;
  const int64_t b = pair / gamma;
  const int i = int(pair - b * gamma);
  const int64_t jt = alpha_target_row(p, b, i), jd = jt + p.tgt_rows;  // rows of the partials
  const int nvalid = chunk_valid(V, c);
  RawChunk<T, VW> rt, rd;
  load_raw<T, VW>(static_cast<const T*>(p.tgt) + (b * (gamma + 1) + i) * V + c * kChunk, nvalid,
                  lane, rt);
  load_raw<T, VW>(static_cast<const T*>(p.drf) + (b * gamma + i) * V + c * kChunk, nvalid, lane,
                  rd);
  const float te = effective_temperature(uniform_load(p.temp, b));
  const double Td = te;
  const float kk = log2e_over_t(te);
  const RowStat st_t = uniform_load(p.rowstat, jt), st_d = uniform_load(p.rowstat, jd);
  const RowPart ct = uniform_load(p.part, jt * nchunk + c);
  const RowPart cd = uniform_load(p.part, jd * nchunk + c);
  double acc = 0.0;
  if (st_t.valid && st_d.valid) {  // wave-uniform
    const double A = chunk_scale(ct.m, st_t, Td), Bq = chunk_scale(cd.m, st_d, Td);
    if (A > 0.0 && Bq > 0.0) {  // wave-uniform; otherwise min(p, q) is 0 on the chunk
      float zt[kElemsPerLane], zd[kElemsPerLane];
      unpack_chunk<T, VW>(rt, nvalid, lane, zt);
      unpack_chunk<T, VW>(rd, nvalid, lane, zd);
      const double sc = fmax(A, Bq);
      const float ra = float(A / sc), rb = float(Bq / sc);
      acc = sc * wave_sum(lane_term_sum([&](int e) {
              return fminf(ra * softmax_term(zt[e], ct.m, kk), rb * softmax_term(zd[e], cd.m, kk));
            }));
    }
  }
  if (lane == 0) chunk_sum[w] = acc;
}

__global__ __launch_bounds__(kAlphaBlock) void k_chain_alpha_reduce(ChainParams p,
                                                                   const double* chunk_sum,
                                                                   int64_t pairs, float* out_alpha,
                                                                   int32_t* out_status) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t pair = int64_t(blockIdx.x) * (kAlphaBlock / kWave) + wave_id();
  if (pair >= pairs) return;  // wave-uniform
  const int gamma = p.gamma;
  const int64_t nchunk = p.nchunk;
  const int64_t b = pair / gamma;
  const int64_t jt = alpha_target_row(p, b, int(pair - b * gamma)), jd = jt + p.tgt_rows;
  const double* cs = chunk_sum + pair * nchunk;
  double acc = 0.0;
  for (int64_t c0 = 0; c0 < nchunk; c0 += int64_t(kWave) * kMergeBatch) {
    double v[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int64_t c = c0 + int64_t(k) * kWave + lane;
      v[k] = c < nchunk ? cs[c] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) acc += v[k];
  }
  acc = wave_sum(acc);
  if (lane == 0) {
    const bool valid = uniform_load(p.rowstat, jt).valid && uniform_load(p.rowstat, jd).valid;
    out_alpha[pair] = valid ? float(acc) : NAN;
    if (out_status) {
      const float tb = uniform_load(p.temp, b);
      int bits = valid ? 0 : SV_ROW_NONFINITE;
      if (!(tb > 0.0f && tb < INFINITY)) bits |= SV_ROW_BAD_TEMPERATURE;
      out_status[pair] = bits;
    }
  }
}

// Overlap and reduce launches shared by the standalone acceptance rates and chain verification
// with rates (partials and row statistics already in the workspace).
template <typename T, int VW>
hipError_t launch_alpha_tail(const ChainParams& p, int64_t B, double* chunk_sum,
                             float* out_alpha, int32_t* out_status, hipStream_t s) {
  const int64_t pairs = B * p.gamma;
  const int64_t owaves = pairs * p.nchunk;
  constexpr int wpb = kStreamBlock<T> / kWave;
  hipError_t e = launch_kernel("alpha_overlap", k_chain_alpha<T, VW>,
                               dim3(unsigned((owaves + wpb - 1) / wpb)), dim3(kStreamBlock<T>), s,
                               p, chunk_sum, owaves);
  if (e != hipSuccess) return e;
  constexpr int awpb = kAlphaBlock / kWave;
  return launch_kernel("alpha_reduce", k_chain_alpha_reduce,
                       dim3(unsigned((pairs + awpb - 1) / awpb)), dim3(kAlphaBlock), s, p,
                       chunk_sum, pairs, out_alpha, out_status);
}

template <typename T, int VW>
hipError_t run_alpha(const AlphaArgs& a, hipStream_t s) {
  const AlphaLayout L = alpha_layout(a.B, a.gamma, a.V);
  ChainParams p = {};
  p.tgt = a.target;
  p.drf = a.draft;
  p.temp = a.temperature;
  p.gamma = a.gamma;
  p.tgt_rows = a.gamma;
  p.V = a.V;
  p.nchunk = L.nchunk;
  p.part = reinterpret_cast<RowPart*>(a.ws + L.off_part);
  p.rowstat = reinterpret_cast<RowStat*>(a.ws + L.off_rowstat);
  const int64_t rows = int64_t(a.B) * (2 * a.gamma);
  const int64_t total = rows * L.nchunk;
  const int64_t waves = (total + kUnitsPerWave<T> - 1) / kUnitsPerWave<T>;
  constexpr int wpb = kStreamBlock<T> / kWave;
  hipError_t e = launch_kernel("alpha_sweep", k_chain_sweep<T, VW>,
                               dim3(unsigned((waves + wpb - 1) / wpb)), dim3(kStreamBlock<T>), s,
                               p, total);
  if (e != hipSuccess) return e;
  constexpr int awpb = kAlphaBlock / kWave;
  e = launch_kernel("alpha_merge", k_chain_alpha_merge, dim3(unsigned((rows + awpb - 1) / awpb)),
                    dim3(kAlphaBlock), s, p, rows);
  if (e != hipSuccess) return e;
  return launch_alpha_tail<T, VW>(p, a.B, reinterpret_cast<double*>(a.ws + L.off_chunk_sum),
                                  a.out_alpha, a.out_status, s);
}

// ------------------------------------------------------------------------------------ sampler

// Draft-side sampler, one wave per logit row r: merges the row's chunk partials into (M, S),
// locates the chunk holding u * W from the chunk masses and rescans it in token order (the
// inverse CDF of the bonus draw), and evaluates p(y) in fp64.  Rows with a bad temperature,
// a bad uniform or no softmax take token 0.  For rows of up to 64 * kLocateBatch chunks the
// partials are loaded once and both the merge and the chunk masses come from those registers,
// and z(y) is taken from the rescanned chunk: two dependent memory round trips in all.
template <typename T, int VW>
__global__ __launch_bounds__(kWave) void k_sample_draw(ChainParams p, const float* uni,
                                                      int32_t* out_tokens, float* out_prob,
                                                      int32_t* out_status) {
  constexpr int NB = kLocateBatch;
  const int64_t r = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t V = p.V, nchunk = p.nchunk;
  const T* row = static_cast<const T*>(p.tgt) + r * V;
  const float tb = uniform_load(p.temp, r);
  const float te = effective_temperature(tb);
  const double Td = te;
  const float kk = log2e_over_t(te);
  const float uf = uniform_load(uni, r);
  const RowPart* pp = p.part + r * nchunk;
  const bool held = nchunk <= int64_t(kWave) * NB;  // uniform

  RowStat st;
  double w[NB];  // held rows: mass of chunk lane * NB + i
  if (held) {
    RowPart q[NB];
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t c = int64_t(lane) * NB + i;
      q[i] = c < nchunk ? pp[c] : RowPart{-INFINITY, 0, 0.0};
      mloc = fmaxf(mloc, q[i].m);
    }
    const float m = wave_max(mloc);
    const bool finite_max = (m > -INFINITY) && (m < INFINITY);
    double f[NB], s = 0.0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      f[i] = q[i].m == -INFINITY ? 0.0 : exp((double(q[i].m) - double(m)) / Td);
      s += q[i].s * f[i];  // a NaN partial survives the zero factor
    }
    s = finite_max ? wave_sum(s) : 0.0;
    st = RowStat{m, finite_max && (s > 0.0) && (s < INFINITY), s};
#pragma unroll
    for (int i = 0; i < NB; ++i) w[i] = q[i].s * (f[i] / s);  // q.s * chunk_scale
  } else {
    st = merge_row(pp, nchunk, lane, Td);
  }
  int status = 0;
  if (!(tb > 0.0f && tb < INFINITY)) status |= SV_ROW_BAD_TEMPERATURE;
  if (!(uf >= 0.0f && uf < 1.0f)) status |= SV_ROW_BAD_UNIFORM;
  if (!st.valid) status |= SV_ROW_NONFINITE;
  int64_t y = 0;
  double prob = NAN;
  if (status == 0) {
    const double u = uf;
    const Located at = held ? locate_chunk_held(w, lane, u)
                            : locate_chunk(nchunk, lane, u, [&](int64_t c) {
                                const RowPart q = pp[c];
                                return q.s * chunk_scale(q.m, st, Td);
                              });
    const int nvalid = chunk_valid(V, at.chunk);
    RawChunk<T, VW> raw;
    load_raw<T, VW>(row + at.chunk * kChunk, nvalid, lane, raw);
    const RowPart pc = uniform_load(pp, at.chunk);
    const double scale = chunk_scale(pc.m, st, Td);
    float z[kElemsPerLane];
    unpack_chunk<T, VW>(raw, nvalid, lane, z);
    const double tau_loc = scale > 0.0 ? (u * at.total - at.before) / scale : 0.0;
    y = chunk_scan<VW>(at.chunk, V, lane, tau_loc,
                       [&](int i) { return double(softmax_term(z[i], pc.m, kk)); });
    // z(y) from the lane that holds it: chunk offset o = (j * 64 + l) * VW + t.
    const int o = int(y - at.chunk * kChunk);
    const int slot = (o / (VW * kWave)) * VW + o % VW;
    float zy = z[0];
#pragma unroll
    for (int i = 1; i < kElemsPerLane; ++i) zy = i == slot ? z[i] : zy;
    zy = __shfl(zy, (o / VW) % kWave, kWave);
    prob = exp((double(zy) - double(st.m)) / Td) / st.s;
  }
  if (lane == 0) {
    out_tokens[r] = int32_t(y);
    if (out_prob) out_prob[r] = float(prob);
    if (out_status) out_status[r] = status;
  }
}

template <typename T, int VW>
hipError_t run_sample(const SampleArgs& a, hipStream_t s) {
  const SampleLayout L = sample_layout(a.rows, a.V);
  ChainParams p = {};
  p.tgt = a.logits;
  p.drf = a.logits;
  p.temp = a.temperature;
  p.gamma = 0;
  p.tgt_rows = 1;
  p.V = a.V;
  p.nchunk = L.nchunk;
  p.part = reinterpret_cast<RowPart*>(a.ws + L.off_part);
  const int64_t total = int64_t(a.rows) * L.nchunk;
  const int64_t waves = (total + kUnitsPerWave<T> - 1) / kUnitsPerWave<T>;
  constexpr int wpb = kStreamBlock<T> / kWave;
  hipError_t e = launch_kernel("sample_sweep", k_chain_sweep<T, VW>,
                               dim3(unsigned((waves + wpb - 1) / wpb)), dim3(kStreamBlock<T>), s,
                               p, total);
  if (e != hipSuccess) return e;
  return launch_kernel("sample_draw", k_sample_draw<T, VW>, dim3(unsigned(a.rows)), dim3(kWave),
                       s, p, a.uniforms, a.out_tokens, a.out_prob, a.out_status);
}

// Path choice for chain verification (all three give the same bits):
//   fused   one launch, one workgroup per sequence for every step;
//   finish  the sweep across the chip, then one workgroup per sequence for decide, residual and
//           draw (chain_finish);
//   split   the sweep, then decide, residual and draw as three launches.
// A 1024-thread workgroup (one per CU at its register count) streams about 128 KiB per memory
// round trip.  So the fused path wins when a sequence's rows take at most two such rounds, or
// when 192..256 sequences give every CU a workgroup and together they saturate HBM (the tails of
// some sequences then overlap the sweeps of others).  The finish path wins while a sequence's
// residual re-read (2 * V elements) stays small.  Measured per call, split / finish / fused:
// B = 1, V = 1000 fp32: 20.2 / 15.6 / 13.4 us; B = 64, V = 32000 bf16: 27.2 / 24.7 / 33.8 us;
// B = 256, V = 32000 bf16: 49.5 / 42.1 / 38.9 us; B = 256, gamma = 7, V = 152064 fp32:
// 406.8 / 400.8 / 390.4 us; B = 64, V = 128256 bf16: 48.1 / 54.4 / 103.1 us; B = 1, V = 152064
// fp32: 19.7 / 36.6 / 195.8 us; B = 1024, V = 32000 bf16: 141.4 / 144.0 / 145.0 us.
// Both one-workgroup forms need the sequence's partials and residual masses to fit their LDS
// budget; the rates need the sweep's partials in the workspace, so they take finish where fused
// would be chosen.  SPECVERIFY_CHAIN_PATH=fused, =finish or =split forces a path (for tests and
// measurement; subject to the LDS fit, and fused becomes finish with the rates).
enum class ChainPath { kSplit, kFused, kFinish };

constexpr size_t kFusedMaxLds = 32 * 1024;
constexpr int64_t kFusedMaxSeqBytes = 256 * 1024;    // small rows: fused for B <= 256
constexpr int kChipFillMin = 192, kChipFillMax = 256;  // fused whatever the row size
constexpr int64_t kFinishMaxResidualBytes = 256 * 1024;
constexpr int kFinishMaxBatch = 512;

// Early exit (sv_verify_chain_lazy) pays once the sequences give most CUs work; smaller batches
// take the eager paths, whose outputs agree wherever the early-exit contract fixes them.  Of the
// two forms, one launch per position (staged) pays for wide rows, whose pair of rows one CU would
// read slowly, and one workgroup per sequence for narrow ones, where the launches' fixed cost
// would dominate.  Measured per call (staged / one workgroup / eager): B = 256, gamma = 7,
// V = 152064 fp32: 190 / 225 / 400 us; B = 128, same rows: 134 / 208 / 213 us; B = 1024,
// gamma = 4, V = 32000 bf16: 115 / 118 / 151 us; B = 512, gamma = 7, V = 32000 bf16 with drafts
// close to the target: 125 / 111 / 122 us; B = 64, gamma = 4, V = 128256 bf16: 66 / 102 / 48 us.
// SPECVERIFY_CHAIN_PATH=lazy or staged forces a form (testing).
constexpr int kLazyMinBatch = 128;
constexpr int64_t kStagedMinPairBytes = 256 * 1024;

inline size_t lazy_lds_bytes(int64_t nchunk) {
  return (2 * sizeof(RowPart) + sizeof(double)) * size_t(nchunk);
}

enum class LazyForm { kNone, kOneGroup, kStaged };

// The early-exit form sv_verify_chain_lazy takes (kNone: the eager paths).
inline LazyForm lazy_form(const ChainArgs& a, int64_t nchunk, int units_per_group,
                          size_t elem_bytes) {
  const bool staged_ok =
      int64_t(a.B) * stage_groups(0, a.gamma, nchunk, units_per_group) < int64_t(INT32_MAX);
  const bool group_ok = lazy_lds_bytes(nchunk) <= kFusedMaxLds;
  const char* e = getenv("SPECVERIFY_CHAIN_PATH");
  if (e && strcmp(e, "staged") == 0) return staged_ok ? LazyForm::kStaged : LazyForm::kNone;
  if (e && strcmp(e, "lazy") == 0) return group_ok ? LazyForm::kOneGroup : LazyForm::kNone;
  if (e && (strcmp(e, "fused") == 0 || strcmp(e, "finish") == 0 || strcmp(e, "split") == 0))
    return LazyForm::kNone;
  if (a.B < kLazyMinBatch) return LazyForm::kNone;
  if (2 * a.V * int64_t(elem_bytes) >= kStagedMinPairBytes || !group_ok)
    return staged_ok ? LazyForm::kStaged : LazyForm::kNone;
  return LazyForm::kOneGroup;
}

inline size_t fused_lds_bytes(int gamma, int64_t nchunk) {
  return sizeof(RowPart) * size_t(2 * gamma + 1) * size_t(nchunk) + sizeof(double) * size_t(nchunk);
}

inline ChainPath choose_path(const ChainArgs& a, int64_t nchunk, size_t elem_bytes,
                             bool with_rates) {
  if (fused_lds_bytes(a.gamma, nchunk) > kFusedMaxLds) return ChainPath::kSplit;
  const ChainPath fused = with_rates ? ChainPath::kFinish : ChainPath::kFused;
  const char* e = getenv("SPECVERIFY_CHAIN_PATH");
  if (e && strcmp(e, "fused") == 0) return fused;
  if (e && strcmp(e, "finish") == 0) return ChainPath::kFinish;
  if (e && strcmp(e, "split") == 0) return ChainPath::kSplit;
  const int64_t s = int64_t(elem_bytes);
  if (a.B <= kChipFillMax && int64_t(2 * a.gamma + 1) * a.V * s <= kFusedMaxSeqBytes) return fused;
  if (a.B >= kChipFillMin && a.B <= kChipFillMax) return fused;
  if (a.B <= kFinishMaxBatch && 2 * a.V * s <= kFinishMaxResidualBytes) return ChainPath::kFinish;
  return ChainPath::kSplit;
}

template <typename T, int VW>
hipError_t run_chain(const ChainArgs& a, hipStream_t s) {
  const bool with_rates = a.out_alpha != nullptr;
  const ChainLayout L = chain_layout(a.B, a.gamma, a.V, with_rates);
  ChainParams p;
  p.tgt = a.target;
  p.drf = a.draft;
  p.toks = a.draft_tokens;
  p.uni = a.uniforms;
  p.temp = a.temperature;
  p.gamma = a.gamma;
  p.tgt_rows = a.gamma + 1;
  p.V = a.V;
  p.nchunk = L.nchunk;
  p.part = reinterpret_cast<RowPart*>(a.ws + L.off_part);
  p.rowstat = reinterpret_cast<RowStat*>(a.ws + L.off_rowstat);
  p.seq = reinterpret_cast<SeqDecision*>(a.ws + L.off_seq);
  p.wres = reinterpret_cast<double*>(a.ws + L.off_wres);
  p.out_tokens = a.out_tokens;
  p.out_nacc = a.out_num_accepted;
  p.out_p = a.out_p;
  p.out_q = a.out_q;
  p.out_status = a.out_status;
  p.alive = reinterpret_cast<int32_t*>(a.ws + L.off_alive);
  p.hstat = reinterpret_cast<int32_t*>(a.ws + L.off_hstat);
  p.lz = reinterpret_cast<float*>(a.ws + L.off_lz);

  // The one-element-load forms of the one-workgroup kernel would spill; they take the split path.
  const ChainPath path =
      VW > 1 ? choose_path(a, L.nchunk, sizeof(T), with_rates) : ChainPath::kSplit;
  if constexpr (VW > 1) {
    const LazyForm form =
        a.lazy ? lazy_form(a, L.nchunk, kStageUnits<T>, sizeof(T)) : LazyForm::kNone;
    if (form == LazyForm::kStaged) {
      for (int j = 0; j <= a.gamma + 1; ++j) {
        const int G = stage_groups(j, a.gamma, L.nchunk, kStageUnits<T>);
        const hipError_t e = launch_kernel("chain_stage", k_chain_stage<T, VW>,
                                           dim3(unsigned(int64_t(a.B) * G)),
                                           dim3(kStageBlock), s, p, j, G);
        if (e != hipSuccess) return e;
      }
      const int64_t rtotal = int64_t(a.B) * L.nchunk;
      constexpr int rw = kResidualBlock / kWave;
      const hipError_t e = launch_kernel("chain_residual", k_chain_residual<T, VW>,
                                         dim3(unsigned((rtotal + rw - 1) / rw)),
                                         dim3(kResidualBlock), s, p, rtotal);
      if (e != hipSuccess) return e;
      return launch_kernel("chain_draw", k_chain_draw<T, VW>, dim3(unsigned(a.B)), dim3(kWave), s,
                           p);
    }
    if (form == LazyForm::kOneGroup)
      return launch_kernel_shm("chain_lazy", k_chain_lazy<T, VW>, dim3(unsigned(a.B)),
                               dim3(kFusedBlock), lazy_lds_bytes(L.nchunk), s, p);
    if (path == ChainPath::kFused)
      return launch_kernel_shm("chain_fused", k_chain_fused<T, VW>, dim3(unsigned(a.B)),
                               dim3(kFusedBlock), fused_lds_bytes(a.gamma, L.nchunk), s, p);
  }

  const int64_t total = int64_t(a.B) * (2 * a.gamma + 1) * L.nchunk;
  const int64_t waves = (total + kUnitsPerWave<T> - 1) / kUnitsPerWave<T>;
  constexpr int wpb = kStreamBlock<T> / kWave;
  hipError_t e = launch_kernel("chain_sweep", k_chain_sweep<T, VW>,
                               dim3(unsigned((waves + wpb - 1) / wpb)), dim3(kStreamBlock<T>), s,
                               p, total);
  if (e != hipSuccess) return e;
  if constexpr (VW > 1) {
    if (path == ChainPath::kFinish) {
      e = launch_kernel_shm("chain_finish", k_chain_finish<T, VW>, dim3(unsigned(a.B)),
                            dim3(kFusedBlock), fused_lds_bytes(a.gamma, L.nchunk), s, p);
      if (e != hipSuccess || !with_rates) return e;
      return launch_alpha_tail<T, VW>(p, a.B, reinterpret_cast<double*>(a.ws + L.off_alpha_sum),
                                      a.out_alpha, nullptr, s);
    }
  }
  e = launch_kernel("chain_decide", k_chain_decide<T, VW>, dim3(unsigned(a.B)), dim3(kBlock), s, p);
  if (e != hipSuccess) return e;
  const int64_t rtotal = int64_t(a.B) * L.nchunk;
  constexpr int rw = kResidualBlock / kWave;
  e = launch_kernel("chain_residual", k_chain_residual<T, VW>,
                    dim3(unsigned((rtotal + rw - 1) / rw)), dim3(kResidualBlock), s, p, rtotal);
  if (e != hipSuccess) return e;
  e = launch_kernel("chain_draw", k_chain_draw<T, VW>, dim3(unsigned(a.B)), dim3(kWave), s, p);
  if (e != hipSuccess || !with_rates) return e;
  return launch_alpha_tail<T, VW>(p, a.B, reinterpret_cast<double*>(a.ws + L.off_alpha_sum),
                                  a.out_alpha, nullptr, s);
}

}  // namespace

hipError_t launch_sample(const SampleArgs& a, hipStream_t s) {
  if (a.dtype == SV_F32) return a.vec ? run_sample<float, 4>(a, s) : run_sample<float, 1>(a, s);
  return a.vec ? run_sample<uint16_t, 8>(a, s) : run_sample<uint16_t, 1>(a, s);
}

hipError_t launch_alpha(const AlphaArgs& a, hipStream_t s) {
  if (a.dtype == SV_F32) return a.vec ? run_alpha<float, 4>(a, s) : run_alpha<float, 1>(a, s);
  return a.vec ? run_alpha<uint16_t, 8>(a, s) : run_alpha<uint16_t, 1>(a, s);
}

hipError_t launch_chain(const ChainArgs& a, hipStream_t s) {
  if (a.dtype == SV_F32) return a.vec ? run_chain<float, 4>(a, s) : run_chain<float, 1>(a, s);
  return a.vec ? run_chain<uint16_t, 8>(a, s) : run_chain<uint16_t, 1>(a, s);
}

}  // namespace sv
