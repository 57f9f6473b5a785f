// Greedy token-tree verification kernels (SpecInfer style).
//
// Source: SpecInfer article (abeam.tech, arXiv:2305.09781), sections "基本アイデア"
// (basic idea) and "推論方法" (inference): the large model gives, for every node of
// the token tree in one pass, the token that should follow the sequence ending at
// that node; verification walks from the root along children whose token equals
// that output and appends the agreeing run.  Greedy outputs are per-node argmaxes.
//
// Two launches per call:
//   argmax  the single HBM sweep (launch_argmax_rows): each wave owns one chunk (2048
//           elements) of one node's logit row and writes the chunk maximum over non-NaN entries
//           and the lowest index attaining it.
//   walk    merges the partials into g[u] for every node, validates the parent array, and
//           follows, from the root, the lowest-id child c of the current node u whose token is
//           g[u]; g of the last node reached is the bonus token.  Trees of up to 64 nodes take
//           one wave per tree (k_tree_walk_wave: a lane per node, one ballot per step); larger
//           ones one workgroup per tree with a child table in LDS (next[u], an LDS atomic
//           minimum over the nodes).  All global loads of the tree (partials, parents, tokens)
//           are issued together, so the walk takes one memory round trip before its stores.

#include <math.h>

#include "sv_argmax.h"
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kWalkBlock = 1024;
constexpr int kWalkWaves = kWalkBlock / kWave;
constexpr int kNodesPerThread = kMaxTreeNodes / kWalkBlock;
static_assert(kMaxTreeNodes % kWalkBlock == 0, "walk threads cover the largest tree evenly");

struct TreeParams {
  const void* logits;
  const int32_t* parents;
  const int32_t* node_tokens;
  int n_nodes;
  int64_t V;
  int64_t nchunk;
  ArgPart* part;
  int32_t* out_path;
  int32_t* out_tokens;
  int32_t* out_nacc;
  int32_t* out_g;
  int32_t* out_status;
};

// Walk state in LDS: argmax, token and matching child of every node (the launch sizes the
// dynamic LDS to 3 * n_nodes words), and the tree's status bits.
struct WalkShared {
  int32_t* g;
  int32_t* tok;
  int32_t* next;
  int32_t* flags;
};

// Lanes per node in the partials' merge: the smallest power of two holding the row's chunks,
// at most a wave; a wave merges kWave / G nodes at once.
__device__ __forceinline__ int merge_group(int64_t nchunk) {
  int g = 1;
  while (g < kWave && g < nchunk) g <<= 1;
  return g;
}

// Completes tree t from its chunk partials (all threads of the workgroup).
__device__ void finish_tree(const TreeParams& p, int64_t t, const WalkShared& sh) {
  const int n_nodes = p.n_nodes;
  const int64_t base = t * n_nodes;
  const int64_t nchunk = p.nchunk;
  const int wave = wave_id();
  const int lane = threadIdx.x & (kWave - 1);

  // Parent and token of this thread's nodes u = threadIdx.x + q * kWalkBlock.
  int32_t par[kNodesPerThread], tok[kNodesPerThread];
#pragma unroll
  for (int q = 0; q < kNodesPerThread; ++q) {
    const int u = int(threadIdx.x) + q * kWalkBlock;
    par[q] = u < n_nodes ? p.parents[base + u] : 0;
    tok[q] = u < n_nodes ? p.node_tokens[base + u] : 0;
  }

  // g[u] for every node: G lanes per node, each lane taking chunks sub, sub + G, ...,
  // kMergeBatch loads in flight per lane, then a reduction inside the G-lane group.
  const int G = merge_group(nchunk);
  const int per_wave = kWave / G;
  const int sub = lane & (G - 1);
  int local = 0;
  for (int u0 = wave * per_wave; u0 < n_nodes; u0 += kWalkWaves * per_wave) {
    const int u = u0 + lane / G;
    float best = -INFINITY;
    int32_t bidx = INT32_MAX;
    int anynan = 0;
    if (u < n_nodes) {
      const ArgPart* pp = p.part + (base + u) * nchunk;
      for (int64_t c0 = sub; c0 < nchunk; c0 += int64_t(G) * kMergeBatch) {
        ArgPart r[kMergeBatch];
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) {
          const int64_t c = c0 + int64_t(i) * G;
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
    }
    for (int o = G / 2; o > 0; o >>= 1) {  // xor offsets below G stay inside the group
      const float ov = __shfl_xor(best, o, kWave);
      const int32_t oi = __shfl_xor(bidx, o, kWave);
      anynan |= __shfl_xor(anynan, o, kWave);
      if (arg_better(ov, oi, best, bidx)) {
        best = ov;
        bidx = oi;
      }
    }
    if (sub == 0 && u < n_nodes) {
      const int32_t gu = bidx == INT32_MAX ? 0 : bidx;
      sh.g[u] = gu;
      if (p.out_g) p.out_g[base + u] = gu;
      if (anynan) local |= SV_ROW_NONFINITE;
    }
  }

#pragma unroll
  for (int q = 0; q < kNodesPerThread; ++q) {
    const int u = int(threadIdx.x) + q * kWalkBlock;
    if (u < n_nodes) {
      sh.tok[u] = tok[q];
      sh.next[u] = INT32_MAX;
      if (u == 0 ? par[q] != -1 : (par[q] < 0 || par[q] >= u)) local |= SV_ROW_BAD_TREE;
      if (u > 0 && (tok[q] < 0 || int64_t(tok[q]) >= p.V)) local |= SV_ROW_TOKEN_RANGE;
    }
  }
  if (threadIdx.x == 0) *sh.flags = 0;
  __syncthreads();

  // next[u] = lowest-id child of u whose token is g[u] (edges that break the parent order are
  // left out; a tree holding one is not walked).
  if (local) atomicOr(sh.flags, local);
#pragma unroll
  for (int q = 0; q < kNodesPerThread; ++q) {
    const int u = int(threadIdx.x) + q * kWalkBlock;
    if (u > 0 && u < n_nodes && par[q] >= 0 && par[q] < u && tok[q] == sh.g[par[q]])
      atomicMin(&sh.next[par[q]], u);
  }
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  const int status = *sh.flags;

  int k = 0;
  int u = 0;
  if (!(status & (SV_ROW_BAD_TREE | SV_ROW_TOKEN_RANGE))) {
    // Children have larger ids than their parents, so the walk ends within n_nodes steps.
    for (int c = sh.next[0]; c != INT32_MAX; c = sh.next[c]) {
      ++k;
      if (lane == 0) {
        p.out_path[base + k] = c;
        p.out_tokens[base + k - 1] = sh.tok[c];
      }
      u = c;
    }
  }
  for (int i = lane; i < n_nodes; i += kWave) {
    if (i == 0) p.out_path[base] = 0;
    if (i > k) p.out_path[base + i] = -1;
    if (i == k) p.out_tokens[base + i] = sh.g[u];
    if (i > k) p.out_tokens[base + i] = -1;
  }
  if (lane == 0) {
    p.out_nacc[t] = k;
    if (p.out_status) p.out_status[t] = status;
  }
}

// Trees of at most 64 nodes: one wave per tree, lane u = node u, no LDS and no barrier.  Each
// lane merges its node's chunk partials (all loads in flight together), reads its parent's argmax
// with one cross-lane read, and marks itself matched when its token equals it.  The walk is one
// ballot per step: the lowest matched child of the current node.  Children have larger ids than
// their parents, so the nodes of the accepted path sorted by id are in path order, and a node's
// place on the path is the number of path nodes below its id: every output is written in
// parallel.  The same result as finish_tree: the lowest-id matching child at every step, the
// argmax order of merge_row_argmax, and the same validation and fallback.
constexpr int kWalkWaveBatch = 16;  // partials a lane loads at once

__global__ __launch_bounds__(kWave) void k_tree_walk_wave(TreeParams p) {
  const int64_t t = blockIdx.x;
  const int n = p.n_nodes;
  const int lane = threadIdx.x;
  const int64_t base = t * n;
  const bool live = lane < n;
  const int32_t par = live ? p.parents[base + lane] : 0;
  const int32_t tok = live ? p.node_tokens[base + lane] : 0;

  float best = -INFINITY;
  int32_t bidx = INT32_MAX;
  int anynan = 0;
  if (live) {
    const ArgPart* pp = p.part + (base + lane) * p.nchunk;
    for (int64_t c0 = 0; c0 < p.nchunk; c0 += kWalkWaveBatch) {
      ArgPart r[kWalkWaveBatch];
#pragma unroll
      for (int i = 0; i < kWalkWaveBatch; ++i)
        r[i] = c0 + i < p.nchunk ? pp[c0 + i] : ArgPart{-INFINITY, INT32_MAX, 0, 0};
#pragma unroll
      for (int i = 0; i < kWalkWaveBatch; ++i) {
        if (arg_better(r[i].v, r[i].idx, best, bidx)) {
          best = r[i].v;
          bidx = r[i].idx;
        }
        anynan |= r[i].nan;
      }
    }
  }
  const int32_t g = bidx == INT32_MAX ? 0 : bidx;
  if (p.out_g && live) p.out_g[base + lane] = g;

  const bool bad_tree = live && (lane == 0 ? par != -1 : (par < 0 || par >= lane));
  const bool bad_tok = live && lane > 0 && (tok < 0 || int64_t(tok) >= p.V);
  const int status = (__any(bad_tree) ? SV_ROW_BAD_TREE : 0) |
                     (__any(bad_tok) ? SV_ROW_TOKEN_RANGE : 0) |
                     (__any(anynan) ? SV_ROW_NONFINITE : 0);
  // g of this node's parent (lanes whose parent index is out of range read lane 0; they are
  // either the root or a bad tree, which is not walked).
  const int32_t gp = __shfl(g, (par >= 0 && par < kWave) ? par : 0, kWave);
  const bool match = live && lane > 0 && par >= 0 && par < lane && tok == gp;

  uint64_t path = 0;  // accepted nodes other than the root
  int u = 0, k = 0;
  if (!(status & (SV_ROW_BAD_TREE | SV_ROW_TOKEN_RANGE))) {
    for (;;) {  // at most n - 1 steps: every step moves to a larger node id
      const uint64_t kids = __ballot(match && par == u);
      if (kids == 0) break;
      u = __builtin_ctzll(kids);
      path |= uint64_t(1) << u;
      ++k;
    }
  }
  const int32_t bonus = __shfl(g, u, kWave);
  if (live) {
    if ((path >> lane) & 1) {
      const int pos = __popcll(path & ((uint64_t(1) << lane) - 1));  // 0-based place on the path
      p.out_path[base + pos + 1] = lane;
      p.out_tokens[base + pos] = tok;
    }
    if (lane == 0) p.out_path[base] = 0;
    if (lane > k) {
      p.out_path[base + lane] = -1;
      p.out_tokens[base + lane] = -1;
    }
    if (lane == k) p.out_tokens[base + k] = bonus;
  }
  if (lane == 0) {
    p.out_nacc[t] = k;
    if (p.out_status) p.out_status[t] = status;
  }
}

__global__ __launch_bounds__(kWalkBlock) void k_tree_walk(TreeParams p) {
  extern __shared__ int32_t walk_lds[];
  __shared__ int32_t flags;
  WalkShared sh{walk_lds, walk_lds + p.n_nodes, walk_lds + 2 * p.n_nodes, &flags};
  finish_tree(p, blockIdx.x, sh);
}

template <typename T, int VW>
hipError_t run_tree(const TreeArgs& a, hipStream_t s) {
  const TreeLayout L = tree_layout(a.n_trees, a.n_nodes, a.V);
  TreeParams p;
  p.logits = a.logits;
  p.parents = a.parents;
  p.node_tokens = a.node_tokens;
  p.n_nodes = a.n_nodes;
  p.V = a.V;
  p.nchunk = L.nchunk;
  p.part = reinterpret_cast<ArgPart*>(a.ws + L.off_part);
  p.out_path = a.out_path;
  p.out_tokens = a.out_tokens;
  p.out_nacc = a.out_num_accepted;
  p.out_g = a.out_node_argmax;
  p.out_status = a.out_status;
  const hipError_t e = launch_argmax_rows("tree_argmax", a.logits, a.dtype, a.vec,
                                          int64_t(a.n_trees) * a.n_nodes, a.V, p.part, s);
  if (e != hipSuccess) return e;
  if (a.n_nodes <= kWave)
    return launch_kernel("tree_walk", k_tree_walk_wave, dim3(unsigned(a.n_trees)), dim3(kWave), s,
                         p);
  return launch_kernel_shm("tree_walk", k_tree_walk, dim3(unsigned(a.n_trees)), dim3(kWalkBlock),
                           size_t(3) * sizeof(int32_t) * size_t(a.n_nodes), s, p);
}

}  // namespace

hipError_t launch_tree(const TreeArgs& a, hipStream_t s) {
  if (a.dtype == SV_F32) return a.vec ? run_tree<float, 4>(a, s) : run_tree<float, 1>(a, s);
  return a.vec ? run_tree<uint16_t, 8>(a, s) : run_tree<uint16_t, 1>(a, s);
}

}  // namespace sv
