// Greedy chain verification (zero-temperature speculative decoding).
//
// Source: "投機的デコーディングとは？LLMの回答を高速化する仕組み" (ai-compass.weeybrid.co.jp),
// section 候補の採用と棄却を具体例で見る: the target checks the draft's candidates in order,
// keeps each one that equals its own choice, and replaces the first that differs with its own
// choice; under greedy decoding that choice is the argmax of the target's logits.
//
// Two launches per call:
//   argmax  the single HBM sweep over the B * (gamma + 1) target rows (launch_argmax_rows).
//   decide  one workgroup per sequence merges the partials into g_i for every row (one wave per
//           row), then one wave compares draft token i with g_i in lane i and takes the cut
//           k = number of leading matches with one ballot; it writes [x_0 .. x_{k-1}, g_k].
// No draft logits are read: greedy verification needs only the draft's tokens.

#include "sv_argmax.h"
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kDecideBlock = 1024;
constexpr int kDecideWaves = kDecideBlock / kWave;

struct GreedyParams {
  const int32_t* toks;
  int gamma;
  int64_t V;
  int64_t nchunk;
  const ArgPart* part;
  int32_t* out_tokens;
  int32_t* out_nacc;
  int32_t* out_g;
  int32_t* out_status;
};

__global__ __launch_bounds__(kDecideBlock) void k_greedy_decide(GreedyParams p) {
  __shared__ int32_t g[kMaxGamma + 1];
  __shared__ int32_t nan_rows;
  const int64_t b = blockIdx.x;
  const int gamma = p.gamma;
  const int R = gamma + 1;
  const int wave = wave_id();
  const int lane = threadIdx.x & (kWave - 1);
  if (threadIdx.x == 0) nan_rows = 0;
  __syncthreads();
  for (int i = wave; i < R; i += kDecideWaves) {
    int32_t gi;
    int nan;
    merge_row_argmax(p.part + (b * R + i) * p.nchunk, p.nchunk, lane, &gi, &nan);
    if (lane == 0) {
      g[i] = gi;
      if (p.out_g) p.out_g[b * R + i] = gi;
      if (nan) atomicOr(&nan_rows, 1);
    }
  }
  __syncthreads();
  if (wave != 0) return;

  int status = nan_rows ? SV_ROW_NONFINITE : 0;
  int x = 0;
  bool bad = false;
  if (lane < gamma) {
    x = p.toks[b * gamma + lane];
    bad = (x < 0) || (int64_t(x) >= p.V);
  }
  if (__any(bad)) status |= SV_ROW_TOKEN_RANGE;
  int k = 0;
  if (!(status & SV_ROW_TOKEN_RANGE)) {
    // k = number of leading positions whose draft token equals the target's argmax.
    const uint64_t miss = ~uint64_t(__ballot(lane < gamma && x == g[lane]));
    const int lead = miss == 0 ? kWave : __builtin_ctzll(miss);
    k = lead < gamma ? lead : gamma;
  }
  for (int i = lane; i <= gamma; i += kWave) {
    // i < k <= gamma <= 64 only on the first pass, where lane i holds x_i.
    p.out_tokens[b * R + i] = i < k ? x : (i == k ? g[k] : -1);
  }
  if (lane == 0) {
    p.out_nacc[b] = k;
    if (p.out_status) p.out_status[b] = status;
  }
}

}  // namespace

hipError_t launch_greedy(const GreedyArgs& a, hipStream_t s) {
  const GreedyLayout L = greedy_layout(a.B, a.gamma, a.V);
  ArgPart* part = reinterpret_cast<ArgPart*>(a.ws + L.off_part);
  hipError_t e = launch_argmax_rows("chain_greedy_argmax", a.target, a.dtype, a.vec,
                                    int64_t(a.B) * (a.gamma + 1), a.V, part, s);
  if (e != hipSuccess) return e;
  GreedyParams p;
  p.toks = a.draft_tokens;
  p.gamma = a.gamma;
  p.V = a.V;
  p.nchunk = L.nchunk;
  p.part = part;
  p.out_tokens = a.out_tokens;
  p.out_nacc = a.out_num_accepted;
  p.out_g = a.out_argmax;
  p.out_status = a.out_status;
  return launch_kernel("chain_greedy_decide", k_greedy_decide, dim3(unsigned(a.B)),
                       dim3(kDecideBlock), s, p);
}

}  // namespace sv
