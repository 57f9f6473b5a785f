// Accepted-path KV compaction.
//
// Sources: "論文解説: Speculative Sampling — ドラフトモデルによるLLMデコード高速化"
// (0h-n0.github.io explainer of arXiv:2302.01318), implementation notes, KV cache management
// (KVキャッシュ管理): cache entries of rejected tokens are rolled back; SpecInfer article
// (abeam.tech, arXiv:2305.09781), inference (推論方法): the verified run is appended to the
// sequence.
//
// One launch: an HBM copy.  Block (b, s, t) copies tile t of rows path[b][j] of sequence b's
// speculative block to rows dst_start[b] + j of its cache, for the path slots j = s, s + 8, ...
// up to num_accepted[b]; rows of rejected nodes are never read.  Accepted paths are short (a few
// rows) while the path arrays may be long (a tree's node count), so a fixed 8 slot groups per
// sequence keeps the grid small.  Every block of a sequence validates the sequence's whole path,
// so a sequence with a bad index copies nothing (all-or-nothing).

#include "sv_device.h"
#include "sv_internal.h"
#include "sv_launch.h"

namespace sv {
namespace {


struct KvParams {
  const char* src;
  char* dst;
  int64_t row_bytes;
  int32_t n, src_rows, dst_rows;
  const int32_t* path;
  int32_t path_len;
  const int32_t* num_accepted;
  const int32_t* dst_start;
  int32_t* out_status;
  int32_t max_rows;
  int64_t tiles;  // tiles per row
};

// Whole-path check of sequence b: k in range, destination rows in range, every source row in
// the block.  Returns k, or -1 if the sequence is invalid.
__device__ __forceinline__ int32_t valid_k(const KvParams& p, int64_t b) {
  const int32_t k = uniform_load(p.num_accepted, b);
  const int32_t start = uniform_load(p.dst_start, b);
  if (k < 0 || k > p.max_rows - 1) return -1;
  if (start < 0 || int64_t(start) + k + 1 > p.dst_rows) return -1;
  if (p.path) {
    for (int32_t j = 0; j <= k; ++j) {
      const int32_t r = uniform_load(p.path, b * p.path_len + j);
      if (r < 0 || r >= p.src_rows) return -1;
    }
  }
  return k;
}

template <typename VT>
__global__ __launch_bounds__(kKvBlock) void k_kv_compact(KvParams p) {
  const int64_t blk = blockIdx.x;
  const int64_t per_seq = int64_t(kKvSlots) * p.tiles;
  const int64_t b = blk / per_seq;
  const int64_t rem = blk - b * per_seq;
  const int32_t slot = int32_t(rem / p.tiles);
  const int64_t t = rem - int64_t(slot) * p.tiles;
  const int32_t k = valid_k(p, b);
  if (slot == 0 && t == 0 && threadIdx.x == 0 && p.out_status)
    p.out_status[b] = k < 0 ? SV_ROW_BAD_INDEX : 0;
  const int32_t start = uniform_load(p.dst_start, b);
  const int64_t nvec = p.row_bytes / int64_t(sizeof(VT));
  const int64_t v0 = t * (int64_t(kKvBlock) * kKvVecPerThread);
  for (int32_t j = slot; j <= k; j += kKvSlots) {  // block-uniform; k < 0 copies nothing
    const int32_t r = p.path ? uniform_load(p.path, b * p.path_len + j) : j;
    const VT* src = reinterpret_cast<const VT*>(p.src + (b * p.src_rows + r) * p.row_bytes);
    VT* dst = reinterpret_cast<VT*>(p.dst + (b * p.dst_rows + start + j) * p.row_bytes);
    VT v[kKvVecPerThread];
#pragma unroll
    for (int i = 0; i < kKvVecPerThread; ++i) {
      const int64_t e = v0 + int64_t(i) * kKvBlock + threadIdx.x;
      if (e < nvec) v[i] = __builtin_nontemporal_load(&src[e]);
    }
#pragma unroll
    for (int i = 0; i < kKvVecPerThread; ++i) {
      const int64_t e = v0 + int64_t(i) * kKvBlock + threadIdx.x;
      if (e < nvec) __builtin_nontemporal_store(v[i], &dst[e]);
    }
  }
}

template <typename VT>
hipError_t run(KvParams p, hipStream_t s) {
  const int64_t per_tile = int64_t(kKvBlock) * kKvVecPerThread * int64_t(sizeof(VT));
  p.tiles = ceil_div(p.row_bytes, per_tile);
  const int64_t blocks = int64_t(p.n) * kKvSlots * p.tiles;
  return launch_kernel("kv_compact", k_kv_compact<VT>, dim3(unsigned(blocks)), dim3(kKvBlock), s,
                       p);
}

}  // namespace

hipError_t launch_kv_compact(const KvArgs& a, hipStream_t s) {
  KvParams p;
  p.src = static_cast<const char*>(a.src);
  p.dst = static_cast<char*>(a.dst);
  p.row_bytes = a.row_bytes;
  p.n = a.n;
  p.src_rows = a.src_rows;
  p.dst_rows = a.dst_rows;
  p.path = a.path;
  p.path_len = a.path_len;
  p.num_accepted = a.num_accepted;
  p.dst_start = a.dst_start;
  p.out_status = a.out_status;
  p.max_rows = a.path ? a.path_len : a.src_rows;
  p.tiles = 0;
  const uintptr_t bits = reinterpret_cast<uintptr_t>(a.src) | reinterpret_cast<uintptr_t>(a.dst) |
                         uintptr_t(a.row_bytes);
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  if ((bits & 15u) == 0) return run<u32x4>(p, s);
  if ((bits & 3u) == 0) return run<uint32_t>(p, s);
  return run<uint8_t>(p, s);
}

}  // namespace sv
