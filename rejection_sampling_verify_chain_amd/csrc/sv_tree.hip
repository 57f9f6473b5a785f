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
//   walk    one workgroup per tree merges the partials into g[u] for every node (one wave per
//           node, all partial loads in flight together), validates the parent array, and walks
//           from the root with one wave: at node u a ballot over the nodes finds the lowest-id
//           child c with parent u and token g[u]; it writes the accepted path and tokens, then
//           g of the last accepted node as the bonus token.

#include <math.h>

#include "sv_argmax.h"
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kWalkBlock = 1024;  // walk: one wave per node during the merge

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

// Walk state in LDS, sized by the launch to 3 * n_nodes words: argmax, parent and token of
// every node.  Only the walk workgroup of a tree uses it.
struct WalkShared {
  int32_t* g;
  int32_t* par;
  int32_t* tok;
  int32_t flags;
};

// Completes tree t from its chunk partials (all threads of the workgroup).
__device__ void finish_tree(const TreeParams& p, int64_t t, WalkShared& sh) {
  const int n_nodes = p.n_nodes;
  const int64_t base = t * n_nodes;
  const int64_t nchunk = p.nchunk;
  const int wave = wave_id();
  const int lane = threadIdx.x & (kWave - 1);
  if (threadIdx.x == 0) sh.flags = 0;
  __syncthreads();
  int local = 0;
  for (int u = wave; u < n_nodes; u += kWalkBlock / kWave) {
    int32_t gu;
    int nan;
    merge_row_argmax(p.part + (base + u) * nchunk, nchunk, lane, &gu, &nan);
    if (lane == 0) {
      sh.g[u] = gu;
      if (p.out_g) p.out_g[base + u] = gu;
      if (nan) local |= SV_ROW_NONFINITE;
    }
  }
  for (int u = threadIdx.x; u < n_nodes; u += kWalkBlock) {
    const int32_t pu = p.parents[base + u];
    const int32_t tu = p.node_tokens[base + u];
    sh.par[u] = pu;
    sh.tok[u] = tu;
    if (u == 0 ? pu != -1 : (pu < 0 || pu >= u)) local |= SV_ROW_BAD_TREE;
    if (u > 0 && (tu < 0 || int64_t(tu) >= p.V)) local |= SV_ROW_TOKEN_RANGE;
  }
  if (local) atomicOr(&sh.flags, local);
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  const int status = sh.flags;

  int k = 0;
  int u = 0;
  if (!(status & (SV_ROW_BAD_TREE | SV_ROW_TOKEN_RANGE))) {
    for (;;) {
      const int32_t want = sh.g[u];
      int found = -1;
      for (int b0 = 0; b0 < n_nodes; b0 += kWave) {
        const int i = b0 + lane;
        const bool m = i > 0 && i < n_nodes && sh.par[i] == u && sh.tok[i] == want;
        const uint64_t hit = __ballot(m);
        if (hit) {
          found = b0 + __builtin_ctzll(hit);
          break;
        }
      }
      if (found < 0) break;  // parents precede children, so the walk ends within n_nodes steps
      ++k;
      if (lane == 0) {
        p.out_path[base + k] = found;
        p.out_tokens[base + k - 1] = sh.tok[found];
      }
      u = found;
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

__global__ __launch_bounds__(kWalkBlock) void k_tree_walk(TreeParams p) {
  extern __shared__ int32_t walk_lds[];
  __shared__ WalkShared sh;
  if (threadIdx.x == 0) {
    sh.g = walk_lds;
    sh.par = walk_lds + p.n_nodes;
    sh.tok = walk_lds + 2 * p.n_nodes;
  }
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
  return launch_kernel_shm("tree_walk", k_tree_walk, dim3(unsigned(a.n_trees)), dim3(kWalkBlock),
                           size_t(3) * sizeof(int32_t) * size_t(a.n_nodes), s, p);
}

}  // namespace

hipError_t launch_tree(const TreeArgs& a, hipStream_t s) {
  if (a.dtype == SV_F32) return a.vec ? run_tree<float, 4>(a, s) : run_tree<float, 1>(a, s);
  return a.vec ? run_tree<uint16_t, 8>(a, s) : run_tree<uint16_t, 1>(a, s);
}

}  // namespace sv
