// Chain verification: the device pieces every path shares and the chip-wide sweep kernel --
// softmax partials per chunk, the row merge, the decision, the inverse-CDF draw and the residual
// masses.  Source: "論文解説: Speculative Sampling — ドラフトモデルによるLLMデコード高速化"
// (0h-n0.github.io explainer of arXiv:2302.01318), Step 2 (ステップ2), Step 3 (ステップ3) and the
// modified rejection sampling section (修正付き棄却サンプリング).
//
// Included by sv_chain.hip only: the chain, acceptance-rate and sampler kernels form one
// translation unit, so every kernel template is instantiated and registered once.
#pragma once

namespace sv {
namespace {

constexpr int kBlock = 1024;  // decide: one wave per row of a sequence
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kResidualBlock = 256;  // residual: one chunk per wave
static_assert(kBlock <= kMaxBlock && kResidualBlock <= kMaxBlock, "launch limits of the C ABI");

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
  // Staged early exit only: the batch size; list t of the sequences that reached position t + 1
  // (live + t * B, live_count[t] entries, in no fixed order); the checks that need no logit row
  // [B]; the last position each sequence reached [B]; and the drafted tokens' target and draft
  // logits [B][gamma][2].
  int64_t B = 0;
  int32_t* live_count = nullptr;
  int32_t* live = nullptr;
  int32_t* hstat = nullptr;
  int32_t* reached = nullptr;
  float* lz = nullptr;
  // chain_finish over several workgroups per sequence: arrival counts [B], zeroed by the sweep.
  int32_t* arrive = nullptr;
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
    if (hit) return c * kChunk + lane_read(cand, int(__builtin_ctzll(hit)));
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
                                         const Drafted& g, float tb, double Td, int lane,
                                         bool write = true) {
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
      if (write && p.out_p) p.out_p[b * gamma + lane] = float(pi);
      if (write && p.out_q) p.out_q[b * gamma + lane] = float(qi);
    }
    // k = number of leading ones of the accept mask.
    const uint64_t rej = ~uint64_t(__ballot(accept && lane < gamma));
    const int lead = rej == 0 ? kWave : __builtin_ctzll(rej);
    k = lead < gamma ? lead : gamma;
  } else if (write && lane < gamma) {
    if (p.out_p) p.out_p[b * gamma + lane] = NAN;
    if (p.out_q) p.out_q[b * gamma + lane] = NAN;
  }
  // Accepted prefix and padding.  Position k is the draw's alone (chain_finish's several-workgroup
  // form draws in another workgroup, whose store no store here may follow).
  for (int i = lane; write && i <= gamma; i += kWave) {
    if (i == k && !fallback) continue;
    int32_t v = -1;
    if (i < k) v = g.x;  // i < k <= gamma <= 64 only on the first pass, where lane i holds x_i
    if (fallback && i == 0) v = 0;
    p.out_tokens[b * (gamma + 1) + i] = v;
  }
  if (write && fallback && lane == 0) {
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
    ls_state.at = Located{lane_read(cand, L), wave_broadcast(cand_before, L), total};
  }
  const uint64_t pos = __ballot(lp >= 0);
  if (pos) {
    const int L = 63 - __builtin_clzll(pos);
    ls_state.last_c = lane_read(lp, L);
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

// Hand-off between the workgroups of one sequence in chain_finish's several-workgroup form,
// within one launch and without a fence.  A wave publishes a chunk mass with an agent-scope
// atomic exchange and waits for it to return, so it has been performed where the atomics of
// every XCD meet before the workgroup's arrival is counted (an agent-scope atomic add after a
// workgroup barrier).  The workgroup whose arrival completes the count draws, reading the masses
// back with agent-scope atomic read-modify-writes (fetch-or 0), which are performed after that
// last arrival and so return every published value.  Every access to the masses and the counts
// in the launch is atomic; the counts were zeroed by the sweep, the launch before.
__device__ __forceinline__ void publish_mass(double* dst, double v) {
  const uint64_t old = __hip_atomic_exchange(reinterpret_cast<uint64_t*>(dst),
                                             __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("" ::"v"(old) : "memory");  // the returned value is waited on here
}

__device__ __forceinline__ double read_published(double* src) {
  return __builtin_bit_cast(double,
                            __hip_atomic_fetch_or(reinterpret_cast<uint64_t*>(src), uint64_t(0),
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

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

// Row statistics and partials from LDS, residual masses published by the sequence's workgroups.
struct LdsPublishedSrc {
  const RowStat* st;   // [2 * gamma + 1]
  const RowPart* prt;  // [2 * gamma + 1][nchunk]
  double* wr;          // [nchunk], in the workspace
  int64_t nchunk;
  __device__ RowStat stat(int j) const { return st[j]; }
  __device__ RowPart part(int j, int64_t c) const { return prt[j * nchunk + c]; }
  __device__ RowPart part_lane(int j, int64_t c) const { return prt[j * nchunk + c]; }
  __device__ double wres(int64_t c) const { return read_published(wr + c); }
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

// ------------------------------------------------------------------------------------ shared kernels

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
        if (p.arrive != nullptr && k.j == 0 && k.c == 0 && lane == 0) p.arrive[k.b] = 0;
      });
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

// Workgroup of the one-workgroup-per-sequence kernels (fused, finish, early exit).
constexpr int kFusedBlock = 1024;
constexpr int kFusedWaves = kFusedBlock / kWave;
template <typename T>
constexpr int kFusedUnits = kUnitsPerWave<T>;  // chunks per wave in flight

}  // namespace
}  // namespace sv
