// Chain verification with early exit (sv_verify_chain_lazy): the one-workgroup form and the
// staged form.  Source: the Speculative Sampling explainer (0h-n0.github.io, arXiv:2302.01318),
// Step 3 (ステップ3): the tests run in position order and stop at the first rejection.
//
// Included by sv_chain.hip only: the chain, acceptance-rate and sampler kernels form one
// translation unit, so every kernel template is instantiated and registered once.
#pragma once

namespace sv {
namespace {

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
// The positions in order with the whole chip on each.  For position j a sweep launch
// (chain_stage) streams row pair j (target row gamma alone at j = gamma, the bonus row) of every
// sequence that reached position j into chunk partials, in workgroups that each take a slice of
// its chunks, and fetches the drafted token's two logits at j; then a decision launch
// (chain_stage_decide, one workgroup per sequence) merges the pair's partials, tests position j,
// writes the outputs and, at a cut or the bonus row, the decision and row statistics.  The
// sequences that accept join a list in the workspace (an atomic add per sequence), and the next
// sweep and decision take that list: their grids cover the whole batch, the leading workgroups
// take the listed sequences and the rest exit at once.  Launch 0 also checks the inputs that need
// no logit row.  Few sequences are left after the first positions, and a launch that sweeps one
// pair for them is mostly fixed cost, so from position kStageTailFrom on (when gamma >
// kStageTailFrom) one sweep launch takes every remaining row of the sequences still in (pairs
// kStageTailFrom .. gamma - 1 and the bonus row).  The multi-kernel path's residual and draw
// kernels then finish every sequence: the residual launch first tests those last positions in
// order (finish_pending: every wave of such a sequence takes the decisions from the chunk
// partials itself, and the chunk-0 wave writes them), then takes the residual masses of the cut.
// Rows after the cut are read only by that last sweep and never change a result, and each step
// calls the eager path's device functions on the same values, so the outputs agree with
// sv_verify_chain bit for bit (p and q after the cut excepted).

constexpr int kStageBlock = 256;
constexpr int kStageWavesPerSimd = 8;
// First position whose sweep takes all the remaining rows (see above); that launch keeps two
// chunks per wave in flight, at the occupancy their registers allow.  Measured on 256 sequences
// of gamma = 7, V = 152064 fp32 (mean accepted 0.56) per call, with the decisions in their own
// launches: all remaining rows from position 3 on 173.8-174.7 us, from position 4 on 178.9 us,
// from position 5 on 183.3 us (and, with the decisions inside the sweeps, one launch per
// position 187.6-188.0 us, from position 2 on 191.9-192.6 us).
constexpr int kStageTailFrom = 3;
constexpr int kStageTailWavesPerSimd = 4;
static_assert(kStageTailFrom <= kStageLists,
              "the sweeps and decisions of positions 1 .. kStageTailFrom read lists "
              "0 .. kStageTailFrom - 1 of the workspace");

// The position whose sweep takes all the remaining rows, or gamma + 2 (none) for short drafts.
inline int stage_tail(int gamma) { return gamma > kStageTailFrom ? kStageTailFrom : gamma + 2; }
template <typename T>
constexpr int kStageUnits = (kStageBlock / kWave) * kUnitsPerWave<T>;  // chunks per workgroup

// Workgroups per sequence in the sweep of position j <= gamma: one slice of row pair j each (of
// target row gamma alone at j = gamma); the sweep of all remaining rows strides over them.
inline int stage_groups(int j, int gamma, int64_t nchunk, int units_per_group) {
  const int64_t units = (j < gamma ? 2 : 1) * nchunk;
  return int((units + units_per_group - 1) / units_per_group);
}

// Decision of position i of sequence b (i == gamma: the bonus row) from the merged statistics of
// target row i (a) and draft row i (d), with the drafted token's logits fetched earlier into lz
// (one wave; the eager path's arithmetic).  lead: write the outputs, and at a cut or the bonus row
// the decision and row statistics.  Returns whether the sequence goes on to position i + 1; when
// it does not, *stop (if given) receives the decision.
__device__ bool stage_decide(const ChainParams& p, int64_t b, int i, const RowStat& a,
                             const RowStat& d, int status, double Td, bool lead, int lane,
                             SeqDecision* stop = nullptr) {
  const int gamma = p.gamma;
  const int R = 2 * gamma + 1;
  if (!a.valid || !d.valid) status |= SV_ROW_NONFINITE;
  if (status != 0) {
    const SeqDecision dec{0, kDrawNone, status, 0};
    if (lead) {
      write_fallback(p, b, status, lane);
      if (lane == 0) p.seq[b] = dec;
    }
    if (stop) *stop = dec;
    return false;
  }
  if (i == gamma) {
    const SeqDecision dec{gamma, kDrawBonus, 0, 0};
    if (lead && lane == 0) {
      p.rowstat[b * R + gamma] = a;
      p.seq[b] = dec;
    }
    if (stop) *stop = dec;
    return false;
  }
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
  if (!accept && stop) *stop = SeqDecision{i, kDrawResidual, 0, 0};
  return accept;
}

// Positions s .. gamma of sequence b, which reached position s in the staged early exit's last
// sweep (every remaining row swept, none tested yet), tested in order from the chunk partials (one
// wave; each step as the decision launches take it).  lead: write the outputs, decision and row
// statistics.  Returns the decision; at a cut, at and ad receive the cut pair's statistics.
__device__ SeqDecision finish_pending(const ChainParams& p, int64_t b, int s, bool lead, int lane,
                                      RowStat& at, RowStat& ad) {
  const int gamma = p.gamma;
  const int R = 2 * gamma + 1;
  const double Td = effective_temperature(uniform_load(p.temp, b));
  for (int i = s;; ++i) {  // wave-uniform; stage_decide stops at i == gamma at the latest
    const RowStat a = merge_row(p.part + (b * R + i) * p.nchunk, p.nchunk, lane, Td);
    const RowStat d =
        i < gamma ? merge_row(p.part + (b * R + gamma + 1 + i) * p.nchunk, p.nchunk, lane, Td) : a;
    SeqDecision stop;
    if (!stage_decide(p, b, i, a, d, 0, Td, lead, lane, &stop)) {
      at = a;
      ad = d;
      return stop;
    }
  }
}

// The drafted tokens' two logits at positions i = i0 + lane, i0 + lane + 64, ... < i1 (one wave),
// for the decisions of those positions.
template <typename T>
__device__ __forceinline__ void fetch_drafted(const ChainParams& p, int64_t b, int i0, int i1,
                                              int lane) {
  const T* tgt = static_cast<const T*>(p.tgt);
  const T* drf = static_cast<const T*>(p.drf);
  for (int i = i0 + lane; i < i1; i += kWave) {
    const int x = p.toks[b * p.gamma + i];
    if (x >= 0 && int64_t(x) < p.V) {
      p.lz[(b * p.gamma + i) * 2] = widen(chain_row(tgt, drf, b, p.gamma, i, p.V)[x]);
      p.lz[(b * p.gamma + i) * 2 + 1] =
          widen(chain_row(tgt, drf, b, p.gamma, p.gamma + 1 + i, p.V)[x]);
    }
  }
}

// Sweep launch j: pair j (target row gamma alone at j = gamma) of every sequence that reached
// position j, or with TAIL every row it still has (pairs j .. gamma - 1 and the bonus row), in
// G workgroups per sequence.  Launch 0 takes every sequence, checks the inputs that need no logit
// row and empties the lists; launch j > 0 takes list j - 1, its leading workgroups working and
// those past the list's end exiting at once.  The lead workgroup also fetches the drafted
// tokens' two logits at the positions it sweeps, for their decisions.
template <typename T, int VW, bool TAIL>
__global__ __launch_bounds__(kStageBlock, TAIL ? kStageTailWavesPerSimd : kStageWavesPerSimd) void
k_chain_stage(ChainParams p, int j, int G) {
  const int64_t rank = blockIdx.x / G;
  const int g = int(blockIdx.x - rank * G);
  int64_t b = rank;
  if (j >= 1) {
    const int32_t listed = uniform_load(p.live, (j - 1) * p.B + rank);  // rank < B: in the list
    if (rank >= uniform_load(p.live_count, j - 1)) return;  // the whole workgroup
    b = listed;
  }
  const bool lead = g == 0;
  const int gamma = p.gamma;
  const int R = 2 * gamma + 1;
  const int64_t nchunk = p.nchunk;
  const int wave = wave_id();
  const int lane = threadIdx.x & (kWave - 1);
  const T* tgt = static_cast<const T*>(p.tgt);
  const T* drf = static_cast<const T*>(p.drf);
  const float tb = uniform_load(p.temp, b);
  const float kk = log2e_over_t(effective_temperature(tb));

  if (j == 0) {
    if (lead && wave == 0) {
      // Checks that read no logit row; the decision of position 0 takes the fallback on them.
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
        p.reached[b] = 0;
      }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0)  // the lists start empty each call
      for (int t = 0; t < kStageLists; ++t) p.live_count[t] = 0;
  }

  constexpr int U = kUnitsPerWave<T>;
  const int64_t u0 = int64_t(g) * kStageUnits<T> + int64_t(wave) * U;
  if (TAIL) {
    // Every remaining row: pairs j .. gamma - 1, then the bonus row, G workgroups striding over
    // their chunks; the drafted tokens' logits of positions j .. gamma - 1.
    static_assert(U == 1, "the stride below gives each wave one unit per step");
    if (lead && wave == 0) fetch_drafted<T>(p, b, j, gamma, lane);
    const int64_t pair_units = int64_t(gamma - j) * 2 * nchunk;
    const int64_t units = pair_units + nchunk;
    const int64_t stride = int64_t(G) * kStageUnits<T>;
    auto where = [&](int64_t w, int& row, int64_t& c) {
      if (w < pair_units) {
        const int64_t q = w / (2 * nchunk), rem = w - q * 2 * nchunk;
        row = rem < nchunk ? j + int(q) : gamma + 1 + j + int(q);
        c = rem < nchunk ? rem : rem - nchunk;
      } else {
        row = gamma;
        c = w - pair_units;
      }
    };
    // Two chunks per wave in flight: the next one's loads go out before this one is reduced.
    for (int64_t w = u0; w < units; w += 2 * stride) {  // wave-uniform
      int row0, row1;
      int64_t c0, c1;
      const int64_t w1 = w + stride < units ? w + stride : w;  // the last odd one reloads w
      where(w, row0, c0);
      where(w1, row1, c1);
      RawChunk<T, VW> r0, r1;
      load_raw<T, VW>(chain_row(tgt, drf, b, gamma, row0, p.V) + c0 * kChunk,
                      chunk_valid(p.V, c0), lane, r0);
      load_raw<T, VW>(chain_row(tgt, drf, b, gamma, row1, p.V) + c1 * kChunk,
                      chunk_valid(p.V, c1), lane, r1);
      float z[kElemsPerLane];
      unpack_chunk<T, VW>(r0, chunk_valid(p.V, c0), lane, z);
      RowPart rp = reduce_chunk(z, kk);
      if (lane == 0) p.part[(b * R + row0) * nchunk + c0] = rp;
      if (w1 != w) {
        unpack_chunk<T, VW>(r1, chunk_valid(p.V, c1), lane, z);
        rp = reduce_chunk(z, kk);
        if (lane == 0) p.part[(b * R + row1) * nchunk + c1] = rp;
      }
    }
    return;
  }
  // The drafted token's logits at position j, for its decision.
  if (lead && wave == 0 && j < gamma) fetch_drafted<T>(p, b, j, j + 1, lane);
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

// Decision of position i (i == gamma: the bonus row) for every sequence that reached it (all at
// i = 0, else list i - 1), one workgroup each: waves 0 and 1 merge the chunk partials of target
// row i and draft row i, and wave 0 decides and writes the outputs.  A sequence that accepts
// (i < gamma) joins list i, which the next sweep launch and decision take.
constexpr int kStageDecideBlock = 2 * kWave;
__global__ __launch_bounds__(kStageDecideBlock) void k_chain_stage_decide(ChainParams p, int i) {
  __shared__ RowStat st2[2];
  const int64_t rank = blockIdx.x;
  int64_t b = rank;
  if (i >= 1) {
    const int32_t listed = uniform_load(p.live, (i - 1) * p.B + rank);  // rank < B: in the list
    if (rank >= uniform_load(p.live_count, i - 1)) return;  // the whole workgroup
    b = listed;
  }
  const int gamma = p.gamma;
  const int R = 2 * gamma + 1;
  const int wave = wave_id();
  const int lane = threadIdx.x & (kWave - 1);
  const double Td = effective_temperature(uniform_load(p.temp, b));
  if (wave < (i < gamma ? 2 : 1)) {
    const RowStat st = merge_row(p.part + (b * R + (wave == 0 ? i : gamma + 1 + i)) * p.nchunk,
                                 p.nchunk, lane, Td);
    if (lane == 0) st2[wave] = st;
  }
  __syncthreads();
  if (wave != 0) return;
  const RowStat a = st2[0];
  const RowStat d = i < gamma ? st2[1] : a;
  const int status = i == 0 ? uniform_load(p.hstat, b) : 0;
  if (stage_decide(p, b, i, a, d, status, Td, true, lane) && lane == 0) {
    // Reached position i + 1: list i.
    p.reached[b] = i + 1;
    if (i < kStageLists) {
      const int32_t at = __hip_atomic_fetch_add(&p.live_count[i], 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      p.live[i * p.B + at] = int32_t(b);
    }
  }
}

}  // namespace
}  // namespace sv
