// Greedy token-tree verification kernels (SpecInfer style).
//
// Source: SpecInfer article (abeam.tech, arXiv:2305.09781), sections "基本アイデア"
// (basic idea) and "推論方法" (inference): the large model gives, for every node of
// the token tree in one pass, the token that should follow the sequence ending at
// that node; verification walks from the root along children whose token equals
// that output and appends the agreeing run.  Greedy outputs are per-node argmaxes.
//
// Pipeline:
//   1. argmax  one wave per (node row, chunk): chunk maximum over non-NaN entries and
//              the lowest index attaining it.  The single HBM sweep over all logits.
//   2. walk    one workgroup per tree: merge chunk partials into g[u] for every node,
//              validate the parent array, then one wave walks from the root: at node u
//              a ballot over the nodes finds the lowest-id child c with parent u and
//              token g[u]; the accepted path and tokens are written, then g of the last
//              accepted node as the bonus token.

#include <math.h>

#include "sv_device.h"
#include "sv_internal.h"
#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

template <typename T, int VW>
__global__ __launch_bounds__(kBlock) void k_tree_argmax(const T* __restrict__ logits, int64_t V,
                                                        int64_t nchunk, int64_t total,
                                                        ArgPart* __restrict__ part) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t w = int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x / kWave);
  if (w >= total) return;
  const int64_t row = w / nchunk;
  const int64_t c = w - row * nchunk;

  float z[kElemsPerLane];
  load_chunk<T, VW>(logits + row * V, V, c, lane, z);

  float m = -INFINITY;
  bool nan = false;
#pragma unroll
  for (int i = 0; i < kElemsPerLane; ++i) {
    m = fmaxf(m, z[i]);  // NaN never wins
    nan |= (z[i] != z[i]);
  }
  m = wave_max(m);
  // Lowest element index holding m: within a lane, (j, t) order is increasing index.
  int idx = INT32_MAX;
#pragma unroll
  for (int j = kElemsPerLane / VW - 1; j >= 0; --j) {
#pragma unroll
    for (int t = VW - 1; t >= 0; --t) {
      const int off = chunk_offset<VW>(j, lane, t);
      if (z[j * VW + t] == m && c * kChunk + off < V) idx = off;
    }
  }
  idx = wave_min(idx);
  const int any_nan = __any(nan);
  if (lane == 0) {
    part[w] = ArgPart{m, idx == INT32_MAX ? INT32_MAX : int32_t(c * kChunk + idx), any_nan, 0};
  }
}

__global__ __launch_bounds__(kBlock) void k_tree_walk(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ node_tokens, int n_nodes,
    int64_t V, int64_t nchunk, const ArgPart* __restrict__ part, int32_t* __restrict__ out_path,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_nacc,
    int32_t* __restrict__ out_g, int32_t* __restrict__ out_status) {
  __shared__ int32_t g[kMaxTreeNodes];
  __shared__ int32_t par[kMaxTreeNodes];
  __shared__ int32_t tok[kMaxTreeNodes];
  __shared__ int32_t flags;
  const int64_t t = blockIdx.x;
  const int64_t base = t * n_nodes;
  if (threadIdx.x == 0) flags = 0;
  __syncthreads();

  int local = 0;
  for (int u = threadIdx.x; u < n_nodes; u += kBlock) {
    const ArgPart* pp = part + (base + u) * nchunk;
    float best = -INFINITY;
    int32_t bidx = INT32_MAX;
    int nan = 0;
    for (int64_t c = 0; c < nchunk; ++c) {
      const ArgPart a = pp[c];
      if (a.v > best || (a.v == best && a.idx < bidx)) {
        best = a.v;
        bidx = a.idx;
      }
      nan |= a.nan;
    }
    const int32_t gu = bidx == INT32_MAX ? 0 : bidx;
    const int32_t pu = parents[base + u];
    const int32_t tu = node_tokens[base + u];
    g[u] = gu;
    par[u] = pu;
    tok[u] = tu;
    if (out_g) out_g[base + u] = gu;
    if (nan) local |= SV_ROW_NONFINITE;
    if (u == 0 ? pu != -1 : (pu < 0 || pu >= u)) local |= SV_ROW_BAD_TREE;
    if (u > 0 && (tu < 0 || int64_t(tu) >= V)) local |= SV_ROW_TOKEN_RANGE;
  }
  if (local) atomicOr(&flags, local);
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  const int status = flags;

  int k = 0;
  int u = 0;
  if (!(status & (SV_ROW_BAD_TREE | SV_ROW_TOKEN_RANGE))) {
    for (;;) {
      const int32_t want = g[u];
      int found = -1;
      for (int b0 = 0; b0 < n_nodes; b0 += kWave) {
        const int i = b0 + lane;
        const bool m = i > 0 && i < n_nodes && par[i] == u && tok[i] == want;
        const uint64_t hit = __ballot(m);
        if (hit) {
          found = b0 + __builtin_ctzll(hit);
          break;
        }
      }
      if (found < 0) break;  // parents precede children, so the walk ends within n_nodes steps
      ++k;
      if (lane == 0) {
        out_path[base + k] = found;
        out_tokens[base + k - 1] = tok[found];
      }
      u = found;
    }
  }
  for (int i = lane; i < n_nodes; i += kWave) {
    if (i == 0) out_path[base] = 0;
    if (i > k) out_path[base + i] = -1;
    if (i == k) out_tokens[base + i] = g[u];
    if (i > k) out_tokens[base + i] = -1;
  }
  if (lane == 0) {
    out_nacc[t] = k;
    if (out_status) out_status[t] = status;
  }
}

template <typename T, int VW>
hipError_t run_tree(const TreeArgs& a, hipStream_t s) {
  const TreeLayout L = tree_layout(a.n_trees, a.n_nodes, a.V);
  ArgPart* part = reinterpret_cast<ArgPart*>(a.ws + L.off_part);
  const int64_t total = int64_t(a.n_trees) * a.n_nodes * L.nchunk;
  hipError_t e = launch_kernel("tree_argmax", k_tree_argmax<T, VW>,
                               dim3(unsigned((total + kWavesPerBlock - 1) / kWavesPerBlock)),
                               dim3(kBlock), s, static_cast<const T*>(a.logits), a.V, L.nchunk,
                               total, part);
  if (e != hipSuccess) return e;
  return launch_kernel("tree_walk", k_tree_walk, dim3(unsigned(a.n_trees)), dim3(kBlock), s, a.parents,
                       a.node_tokens, a.n_nodes, a.V, L.nchunk, (const ArgPart*)part, a.out_path,
                       a.out_tokens, a.out_num_accepted, a.out_node_argmax, a.out_status);
}

}  // namespace

hipError_t launch_tree(const TreeArgs& a, hipStream_t s) {
  if (a.dtype == SV_F32) return a.vec ? run_tree<float, 4>(a, s) : run_tree<float, 1>(a, s);
  return a.vec ? run_tree<uint16_t, 8>(a, s) : run_tree<uint16_t, 1>(a, s);
}

}  // namespace sv
