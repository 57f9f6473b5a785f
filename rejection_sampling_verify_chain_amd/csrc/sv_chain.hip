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
// Layout: sv_chain_common.h holds the device pieces every path shares (softmax partials, row
// merge, decision, inverse-CDF draw, residual masses) and the sweep kernel;
// sv_chain_early_exit.h the two early-exit forms; sv_chain_rates.h the per-position acceptance
// rates and sv_chain_sample.h the draft-side sampler, which reuse the sweep, the row merge and
// the draw.  This file holds the split and one-workgroup paths, the path choice and the entry
// functions.  All of them form this one translation unit.

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "sv_device.h"
#include "sv_internal.h"
#include "sv_launch.h"
#include "sv_chain_common.h"
#include "sv_chain_early_exit.h"
#include "sv_chain_rates.h"
#include "sv_chain_sample.h"

namespace sv {
namespace {

// ------------------------------------------------------------------------------------ kernels

template <typename T, int VW>
__global__ __launch_bounds__(kBlock) void k_chain_decide(ChainParams p) {
  __shared__ DecideShared sh;
  decide_sequence<T, VW>(p, blockIdx.x, sh);
}

// The wave's chunk loads of both rows are issued as soon as the decision (which row) is known;
// the chunk partials and row statistics that scale them arrive through the scalar cache while
// the chunk is in flight.  A chunk whose target part is all -inf (A = 0) is loaded too and adds
// nothing.  PENDING (the staged early exit's form): a sequence that reached position `pending` in
// the last sweep has no decision yet; each of its waves takes the decisions from the chunk
// partials itself (finish_pending; the chunk-0 wave writes them), with the cut pair's statistics
// in hand.  The other forms keep the plain kernel (one fewer dependent load ahead of the rows).
template <typename T, int VW, bool PENDING>
__global__ __launch_bounds__(kResidualBlock) void k_chain_residual(ChainParams p, int64_t total,
                                                                   int pending) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t w = int64_t(blockIdx.x) * (kResidualBlock / kWave) + wave_id();
  if (w >= total) return;  // wave-uniform
  const int64_t b = w / p.nchunk;
  const int64_t c = w - b * p.nchunk;
  const bool decide_here = PENDING && uniform_load(p.reached, b) == pending;
  RowStat st_t{}, st_d{};
  SeqDecision d;
  if (decide_here)
    d = finish_pending(p, b, pending, c == 0, lane, st_t, st_d);
  else
    d = uniform_load(p.seq, b);
  if (d.mode != kDrawResidual) return;
  const int R = 2 * p.gamma + 1;
  const int jt = d.k, jd = p.gamma + 1 + d.k;
  const T* tgt = static_cast<const T*>(p.tgt);
  const T* drf = static_cast<const T*>(p.drf);
  const int nvalid = chunk_valid(p.V, c);
  RawChunk<T, VW> rt, rd;
  load_raw<T, VW>(chain_row(tgt, drf, b, p.gamma, jt, p.V) + c * kChunk, nvalid, lane, rt);
  load_raw<T, VW>(chain_row(tgt, drf, b, p.gamma, jd, p.V) + c * kChunk, nvalid, lane, rd);
  if (!decide_here) {
    st_t = uniform_load(p.rowstat, b * R + jt);
    st_d = uniform_load(p.rowstat, b * R + jd);
  }
  const float te = effective_temperature(uniform_load(p.temp, b));
  const double w_c = residual_chunk_mass<T, VW>(
      rt, rd, nvalid, lane, uniform_load(p.part, (b * R + jt) * p.nchunk + c),
      uniform_load(p.part, (b * R + jd) * p.nchunk + c), st_t, st_d, double(te),
      log2e_over_t(te));
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

struct FusedShared {
  RowStat st[2 * kMaxGamma + 1];
  SeqDecision d;
  int last;
};

// The body of chain_fused and chain_finish (all threads of the sequence's workgroup); fused_lds
// is the launch's dynamic LDS: partials [R][nchunk], then residual masses [nchunk].  With G > 1
// (chain_finish on small batches) G workgroups share each sequence: every one copies and merges
// its partials and takes the decision; the first writes the results; each computes the residual
// masses of every G-th chunk and publishes them (publish_mass), and the last to arrive draws.
// That spreads the residual pass, bound by its two exponentials per element on one compute
// unit, over G of them.
template <typename T, int VW, bool SWEPT, int G>
__device__ __forceinline__ void one_workgroup_chain(const ChainParams& p, unsigned char* fused_lds,
                                                    FusedShared& sh) {
  static_assert(G == 1 || SWEPT, "several workgroups per sequence only after the sweep");
  const int64_t b = G == 1 ? int64_t(blockIdx.x) : int64_t(blockIdx.x / G);
  const int grp = G == 1 ? 0 : int(blockIdx.x % G);
  const bool lead = grp == 0;
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
      if (SWEPT && lead) p.rowstat[b * R + j] = st;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const SeqDecision d = decide_from_stats(p, b, sh.st, g, tb, Td, lane, lead);
    if (lane == 0) sh.d = d;
  }
  __syncthreads();
  const SeqDecision d = sh.d;
  if (d.mode == kDrawNone) return;  // the whole workgroup: the decision wrote the result
  if (d.mode == kDrawResidual) {     // the whole workgroup
    const int jt = d.k, jd = gamma + 1 + d.k;
    for (int64_t c = grp + int64_t(G) * wave; c < nchunk; c += int64_t(G) * kFusedWaves) {
      const int nvalid = chunk_valid(V, c);
      RawChunk<T, VW> rt, rd;
      load_raw<T, VW>(chain_row(tgt, drf, b, gamma, jt, V) + c * kChunk, nvalid, lane, rt);
      load_raw<T, VW>(chain_row(tgt, drf, b, gamma, jd, V) + c * kChunk, nvalid, lane, rd);
      const double w_c = residual_chunk_mass<T, VW>(rt, rd, nvalid, lane, prt[jt * nchunk + c],
                                                    prt[jd * nchunk + c], sh.st[jt], sh.st[jd],
                                                    Td, kk);
      if (lane == 0) {
        if constexpr (G == 1)
          wr[c] = w_c;
        else
          publish_mass(p.wres + b * nchunk + c, w_c);
      }
    }
    __syncthreads();
    if constexpr (G > 1) {
      if (threadIdx.x == 0)
        sh.last = __hip_atomic_fetch_add(p.arrive + b, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == G - 1;
      __syncthreads();
      if (!sh.last) return;  // the whole workgroup
    }
  } else if (!lead) {
    return;  // the bonus draw is the first workgroup's
  }
  if (wave != 0) return;
  if constexpr (G == 1)
    draw_sequence<T, VW>(p, b, d, LdsSrc{sh.st, prt, wr, nchunk});
  else
    draw_sequence<T, VW>(p, b, d, LdsPublishedSrc{sh.st, prt, p.wres + b * nchunk, nchunk});
}

template <typename T, int VW>
__global__ __launch_bounds__(kFusedBlock) void k_chain_fused(ChainParams p) {
  extern __shared__ __align__(16) unsigned char fused_lds[];
  __shared__ FusedShared sh;
  one_workgroup_chain<T, VW, false, 1>(p, fused_lds, sh);
}

template <typename T, int VW, int G>
__global__ __launch_bounds__(kFusedBlock) void k_chain_finish(ChainParams p) {
  extern __shared__ __align__(16) unsigned char fused_lds[];
  __shared__ FusedShared sh;
  one_workgroup_chain<T, VW, true, G>(p, fused_lds, sh);
}

enum class ChainPath { kSplit, kFused, kFinish };

constexpr size_t kFusedMaxLds = 32 * 1024;
constexpr int64_t kFusedMaxSeqBytes = 256 * 1024;    // small rows: fused for B <= 256
constexpr int kChipFillMin = 192, kChipFillMax = 256;  // fused whatever the row size
constexpr int64_t kFinishMaxResidualBytes = 256 * 1024;
constexpr int kFinishMaxBatch = 512;
// Workgroups per sequence in chain_finish: for rows of 16 chunks or more, 4 up to 64 sequences
// and 2 up to 128 (the launch stays within one 1024-thread workgroup per compute unit), else 1.
// With fewer chunks one workgroup's residual pass has at most two chunk pairs per SIMD, and the
// hand-off costs what the split saves.  Measured per call, one workgroup against the split:
// B = 1, gamma = 4, V = 32000 bf16 16.0-16.4 against 13.4-14.1 us; B = 32 19.6 against 17.7 us;
// B = 64 23.1-23.3 against 21.4 us; B = 64, V = 65536 bf16 33.8-33.9 against 28.6-28.8 us;
// B = 96, V = 32000 bf16 26.2 against 25.2 us (2 per sequence); B = 128 29.5-29.6 against
// 28.7-28.8 us; B = 128, V = 65536 bf16 46.3 against 43.9 us; 8-chunk fp32 rows (V = 16384,
// gamma = 7): B = 64 24.9 against 24.9 us, B = 128 34.0 against 34.9 us.
constexpr int kFinishGroupsMinBatch = 16;  // wide rows: chain_finish from here (choose_path)
inline int finish_groups(int B, int64_t nchunk) {
  if (nchunk < 16) return 1;
  return B <= 64 ? 4 : B <= 128 ? 2 : 1;
}

// Early exit (sv_verify_chain_lazy) pays once the batch holds enough rows; smaller batches take
// the eager paths, whose outputs agree wherever the early-exit contract fixes them.  One
// workgroup per sequence pays once every CU has a sequence and the row pairs are narrow (a CU
// reads its sequence's pairs one after another); one launch per position (staged) pays for wide
// pairs, and for narrower ones in large batches.  The gate (lazy_form), with W = B x (bytes of
// one row pair): below kLazyMinBatch sequences eager; pairs of kStagedWidePairBytes or more
// staged; below kLazyGroupBatch sequences staged when W >= kStagedMinFirstPairs, else eager;
// otherwise staged for pairs of kStagedMinPairBytes or more from kStagedBatch sequences on, else
// one workgroup per sequence.  Measured per call (staged / one workgroup / eager): B = 256, gamma = 7,
// V = 152064 fp32: 171 / 223 / 398 us; B = 128, same rows: 113 / 195 / 211 us; B = 256,
// gamma = 7, V = 131072 bf16: 141 / 164 / 209 us; B = 256, gamma = 7, V = 65536 bf16: 105 / 93 /
// 114 us; B = 512, gamma = 4, V = 65536 bf16: 123 / 125 / 151 us; B = 1024, gamma = 4,
// V = 32000 bf16: 134 / 132 / 151 us; B = 64, gamma = 4, V = 128256 bf16: 63 / 102 / 47 us;
// B = 128, gamma = 7, V = 65536 bf16: 75 / 88 / 64 us; B = 128, gamma = 7, V = 98304 bf16:
// 85 / 125 / 91 us; B = 192, gamma = 7, V = 65536 bf16: 84 / 90 / 100 us; B = 384, gamma = 7,
// V = 65536 bf16: 122 / 132 / 168 us; B = 128, gamma = 7, V = 32000 bf16: 62 / 54 / 39 us.
// SPECVERIFY_CHAIN_PATH=lazy or staged forces a form (testing).
constexpr int kLazyMinBatch = 128;
constexpr int kLazyGroupBatch = 256;                        // one workgroup per sequence from here
constexpr int kStagedBatch = 384;                           // staged for mid-width pairs from here
constexpr int64_t kStagedMinPairBytes = 256 * 1024;         // mid-width pairs
constexpr int64_t kStagedWidePairBytes = 512 * 1024;        // wide pairs: staged at any batch
constexpr int64_t kStagedMinFirstPairs = int64_t(48) << 20;  // W below kLazyGroupBatch

inline size_t lazy_lds_bytes(int64_t nchunk) {
  return (2 * sizeof(RowPart) + sizeof(double)) * size_t(nchunk);
}

enum class LazyForm { kNone, kOneGroup, kStaged };

// The early-exit form sv_verify_chain_lazy takes (kNone: the eager paths).
inline LazyForm lazy_form(const ChainArgs& a, int64_t nchunk, int units_per_group,
                          size_t elem_bytes) {
  const bool staged_ok = work_items_fit(
      int64_t(a.B) * stage_groups(0, a.gamma, nchunk, units_per_group), kStageBlock);
  const bool group_ok = lazy_lds_bytes(nchunk) <= kFusedMaxLds;
  const char* e = getenv("SPECVERIFY_CHAIN_PATH");
  if (e && strcmp(e, "staged") == 0) return staged_ok ? LazyForm::kStaged : LazyForm::kNone;
  if (e && strcmp(e, "lazy") == 0) return group_ok ? LazyForm::kOneGroup : LazyForm::kNone;
  if (e && (strcmp(e, "fused") == 0 || strcmp(e, "finish") == 0 || strcmp(e, "split") == 0))
    return LazyForm::kNone;
  if (a.B < kLazyMinBatch) return LazyForm::kNone;
  const int64_t pair = 2 * a.V * int64_t(elem_bytes);
  const LazyForm staged = staged_ok ? LazyForm::kStaged : LazyForm::kNone;
  if (pair >= kStagedWidePairBytes) return staged;
  if (a.B < kLazyGroupBatch)
    return int64_t(a.B) * pair >= kStagedMinFirstPairs ? staged : LazyForm::kNone;
  if ((pair >= kStagedMinPairBytes && a.B >= kStagedBatch) || !group_ok) return staged;
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
  // Wider rows: chain_finish once it spreads over 64 compute units or more with several
  // workgroups per sequence (16 <= B <= 128), else the multi-kernel path.  Measured per call
  // (split / finish): B = 16, gamma = 4, V = 128256 bf16 24.8 / 24.1 us; B = 32 31.7 / 30.3;
  // B = 64 45.4-46.2 / 43.6; B = 64, gamma = 7 62.4 / 60.0; B = 96 60.2 / 59.7; B = 128 75.5 /
  // 73.4; B = 64 and 128, gamma = 4, V = 65536 fp32 43.2 / 40.3 and 70.3 / 67.6; but B = 8,
  // gamma = 7, V = 152064 fp32 29.6 / 32.1 and B = 1 19.0 / 21.2, where the multi-kernel
  // path's residual pass spreads a sequence over the whole chip.
  if (a.B >= kFinishGroupsMinBatch && finish_groups(a.B, nchunk) > 1) return ChainPath::kFinish;
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
  p.B = a.B;
  p.live_count = reinterpret_cast<int32_t*>(a.ws + L.off_live);
  p.live = p.live_count + kStageCountPad;
  p.hstat = reinterpret_cast<int32_t*>(a.ws + L.off_hstat);
  p.reached = reinterpret_cast<int32_t*>(a.ws + L.off_reached);
  p.lz = reinterpret_cast<float*>(a.ws + L.off_lz);

  // The one-element-load forms of the one-workgroup kernel would spill; they take the split path.
  const ChainPath path =
      VW > 1 ? choose_path(a, L.nchunk, sizeof(T), with_rates) : ChainPath::kSplit;
  if constexpr (VW > 1) {
    const LazyForm form =
        a.lazy ? lazy_form(a, L.nchunk, kStageUnits<T>, sizeof(T)) : LazyForm::kNone;
    if (form == LazyForm::kStaged) {
      const int tail = stage_tail(a.gamma);
      for (int j = 0; j <= a.gamma && j <= tail; ++j) {
        const int G = stage_groups(j, a.gamma, L.nchunk, kStageUnits<T>);
        const dim3 grid(unsigned(int64_t(a.B) * G));
        hipError_t e = j == tail ? launch_kernel("chain_stage", k_chain_stage<T, VW, true>, grid,
                                                 dim3(kStageBlock), s, p, j, G)
                                 : launch_kernel("chain_stage", k_chain_stage<T, VW, false>, grid,
                                                 dim3(kStageBlock), s, p, j, G);
        if (e != hipSuccess) return e;
        if (j == tail) break;
        e = launch_kernel("chain_stage_decide", k_chain_stage_decide, dim3(unsigned(a.B)),
                          dim3(kStageDecideBlock), s, p, j);
        if (e != hipSuccess) return e;
      }
      const int64_t rtotal = int64_t(a.B) * L.nchunk;
      constexpr int rw = kResidualBlock / kWave;
      const dim3 rgrid(unsigned(wave_groups(rtotal, rw)));
      const hipError_t e =
          tail <= a.gamma ? launch_kernel("chain_residual", k_chain_residual<T, VW, true>, rgrid,
                                          dim3(kResidualBlock), s, p, rtotal, tail)
                          : launch_kernel("chain_residual", k_chain_residual<T, VW, false>, rgrid,
                                          dim3(kResidualBlock), s, p, rtotal, -1);
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

  const int fg = VW > 1 && path == ChainPath::kFinish ? finish_groups(a.B, L.nchunk) : 1;
  if (fg > 1) p.arrive = p.reached;  // the staged early exit's record, unused here
  const int64_t total = int64_t(a.B) * (2 * a.gamma + 1) * L.nchunk;
  const int64_t waves = (total + kUnitsPerWave<T> - 1) / kUnitsPerWave<T>;
  constexpr int wpb = kStreamBlock<T> / kWave;
  hipError_t e = launch_kernel("chain_sweep", k_chain_sweep<T, VW>,
                               dim3(unsigned(wave_groups(waves, wpb))), dim3(kStreamBlock<T>), s,
                               p, total);
  if (e != hipSuccess) return e;
  if constexpr (VW > 1) {
    if (path == ChainPath::kFinish) {
      const size_t lds = fused_lds_bytes(a.gamma, L.nchunk);
      const dim3 grid(unsigned(a.B * fg));
      e = fg == 4   ? launch_kernel_shm("chain_finish", k_chain_finish<T, VW, 4>, grid,
                                        dim3(kFusedBlock), lds, s, p)
          : fg == 2 ? launch_kernel_shm("chain_finish", k_chain_finish<T, VW, 2>, grid,
                                        dim3(kFusedBlock), lds, s, p)
                    : launch_kernel_shm("chain_finish", k_chain_finish<T, VW, 1>, grid,
                                        dim3(kFusedBlock), lds, s, p);
      if (e != hipSuccess || !with_rates) return e;
      return launch_alpha_tail<T, VW>(p, a.B, reinterpret_cast<double*>(a.ws + L.off_alpha_sum),
                                      a.out_alpha, nullptr, s);
    }
  }
  e = launch_kernel("chain_decide", k_chain_decide<T, VW>, dim3(unsigned(a.B)), dim3(kBlock), s, p);
  if (e != hipSuccess) return e;
  const int64_t rtotal = int64_t(a.B) * L.nchunk;
  constexpr int rw = kResidualBlock / kWave;
  e = launch_kernel("chain_residual", k_chain_residual<T, VW, false>,
                    dim3(unsigned(wave_groups(rtotal, rw))), dim3(kResidualBlock), s, p, rtotal,
                    -1);
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
