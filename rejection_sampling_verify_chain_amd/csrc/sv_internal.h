// Internal declarations shared by the C-ABI layer and the kernel translation units.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "specverify.h"

namespace sv {

// One wavefront (64 lanes) sweeps one "chunk" of a logit row: every lane holds
// kElemsPerLane consecutive-in-vector elements spread over kElemsPerLane/VEC
// coalesced 16-byte loads.  Chunks are the unit of the per-row partial
// statistics kept in the workspace.
constexpr int kWave = 64;
constexpr int kElemsPerLane = 32;
constexpr int kChunk = kWave * kElemsPerLane;  // elements per chunk (2048)
constexpr int kMaxGamma = 64;
constexpr int kMaxTreeNodes = 4096;
constexpr int kMaxBatch = (1 << 22) - 1;  // one 1024-thread workgroup per sequence: < 2^32 work-items

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Per (row, chunk) softmax partial: chunk max m and sum_x exp((z(x) - m) / T) in fp64.
struct __attribute__((aligned(16))) RowPart {
  float m;
  int32_t pad;
  double s;
};

// Per row merged statistics: row max and sum_x exp((z(x) - max) / T).
struct __attribute__((aligned(16))) RowStat {
  float m;
  int32_t valid;
  double s;
};

// How a finished sequence draws its last token.
enum DrawMode : int32_t { kDrawNone = 0, kDrawBonus = 1, kDrawResidual = 2 };

// Per sequence decision taken by the decide kernel for the residual and draw kernels.
struct __attribute__((aligned(16))) SeqDecision {
  int32_t k;       // drafts accepted
  int32_t mode;    // DrawMode
  int32_t status;  // SV_ROW_* bits so far
  int32_t pad;
};

// Per (row, chunk) argmax partial for the tree path.
struct __attribute__((aligned(16))) ArgPart {
  float v;       // chunk maximum over non-NaN entries (-inf if none)
  int32_t idx;   // lowest index attaining it (INT32_MAX if none)
  int32_t nan;   // chunk holds a NaN
  int32_t pad;
};

// Launch limits.  A dispatch holds its grid size in work-items (workgroups x threads) as a
// 32-bit number, so every launch must stay below 2^32 work-items.  The launches of an entry
// point are of two kinds: one wave per chunk (2048 elements) of every logit row it reads, in
// workgroups of at most kMaxChunkWaves waves, and one workgroup of at most kMaxBlock threads per
// sequence, tree or row.  shape_grids_fit bounds both for a shape; the launchers static_assert
// their block sizes against these constants.
constexpr int64_t kMaxWorkItems = (int64_t(1) << 32) - 1;
constexpr int kMaxBlock = 1024;
constexpr int kMaxChunkWaves = kMaxBlock / kWave;

// ceil(a / b) for a >= 0, b > 0, without forming a + b - 1 (no overflow near INT64_MAX).
inline int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }

inline int64_t n_chunks(int64_t V) { return ceil_div(V, kChunk); }

// `groups` workgroups of `threads` threads fit one launch.
inline bool work_items_fit(int64_t groups, int64_t threads) {
  return groups >= 0 && groups <= kMaxWorkItems / threads;
}

// Every launch for `units` sequences (trees, rows) of `rows_per_unit` logit rows of V elements
// fits: the one-wave-per-chunk launches over all units * rows_per_unit * ceil(V / 2048) chunks
// (rounded up to whole workgroups) and one kMaxBlock-thread workgroup per unit.  The caller
// bounds units <= 2^31, rows_per_unit <= 4096 and V <= 2^31 - 1 first, so the product stays
// below 2^63.
inline bool shape_grids_fit(int64_t units, int64_t rows_per_unit, int64_t V) {
  const int64_t chunks = units * rows_per_unit * n_chunks(V);
  return work_items_fit(units, kMaxBlock) && work_items_fit(chunks + kMaxChunkWaves - 1, kWave);
}

// Workgroups of a launch that gives one wave to each of `units` units, `waves_per_group` waves
// per workgroup.
inline int64_t wave_groups(int64_t units, int64_t waves_per_group) {
  return ceil_div(units, waves_per_group);
}

// Lists of the sequences that reached a position, kept by the staged early exit for its launches
// after the first two and for its last step (see stage_tail): counts, padded to 256 bytes, then
// kStageLists lists of B sequence indices.
constexpr int kStageLists = 3;
constexpr int kStageCountPad = 64;  // int32 slots before the lists

// Workspace: per (row, chunk) partials, per row statistics, per sequence decisions, per
// (sequence, chunk) residual masses, and the staged early exit's sequence lists, input checks,
// last positions reached and drafted logits.  Every entry is written before it is read within a call.
// with_rates: also the per (sequence, position, chunk) overlap sums of the acceptance rates.
struct ChainLayout {
  int64_t nchunk;
  size_t off_part, off_rowstat, off_seq, off_wres, off_live, off_hstat, off_reached, off_lz,
      off_alpha_sum,
      total;
};

inline ChainLayout chain_layout(int64_t B, int64_t gamma, int64_t V, bool with_rates = false) {
  ChainLayout L;
  L.nchunk = n_chunks(V);
  const int64_t rows = B * (2 * gamma + 1);
  size_t off = 0;
  L.off_part = off;
  off += align256(sizeof(RowPart) * size_t(rows) * size_t(L.nchunk));
  L.off_rowstat = off;
  off += align256(sizeof(RowStat) * size_t(rows));
  L.off_seq = off;
  off += align256(sizeof(SeqDecision) * size_t(B));
  L.off_wres = off;
  off += align256(sizeof(double) * size_t(B) * size_t(L.nchunk));
  L.off_live = off;  // staged early exit: counts [kStageCountPad], lists [kStageLists][B] int32
  off += align256(sizeof(int32_t) * (kStageCountPad + size_t(kStageLists) * size_t(B)));
  L.off_hstat = off;  // [B] int32
  off += align256(sizeof(int32_t) * size_t(B));
  L.off_reached = off;  // [B] int32
  off += align256(sizeof(int32_t) * size_t(B));
  L.off_lz = off;  // [B][gamma][2] fp32
  off += align256(sizeof(float) * 2 * size_t(B) * size_t(gamma));
  L.off_alpha_sum = off;
  if (with_rates) off += align256(sizeof(double) * size_t(B) * size_t(gamma) * size_t(L.nchunk));
  L.total = off;
  return L;
}

// Workspace: per (row, chunk) argmax partials.
struct TreeLayout {
  int64_t nchunk;
  size_t off_part, total;
};

inline TreeLayout tree_layout(int64_t n_trees, int64_t n_nodes, int64_t V) {
  TreeLayout L;
  L.nchunk = n_chunks(V);
  L.off_part = 0;
  L.total = align256(sizeof(ArgPart) * size_t(n_trees) * size_t(n_nodes) * size_t(L.nchunk));
  return L;
}

// Workspace of the greedy chain path: per (row, chunk) argmax partials of the target rows.
struct GreedyLayout {
  int64_t nchunk;
  size_t off_part, total;
};

inline GreedyLayout greedy_layout(int64_t B, int64_t gamma, int64_t V) {
  GreedyLayout L;
  L.nchunk = n_chunks(V);
  L.off_part = 0;
  L.total = align256(sizeof(ArgPart) * size_t(B) * size_t(gamma + 1) * size_t(L.nchunk));
  return L;
}

// Workspace of the acceptance-rate path: per (row, chunk) softmax partials of target rows
// 0..gamma-1 and draft rows 0..gamma-1 of every sequence.
// Workspace of the acceptance rates: per (row, chunk) softmax partials of target rows
// 0..gamma-1 and draft rows 0..gamma-1, the merged statistics of those rows, and per
// (sequence, position, chunk) overlap sums.
struct AlphaLayout {
  int64_t nchunk;
  size_t off_part, off_rowstat, off_chunk_sum, total;
};

inline AlphaLayout alpha_layout(int64_t B, int64_t gamma, int64_t V) {
  AlphaLayout L;
  L.nchunk = n_chunks(V);
  const size_t rows = size_t(B) * size_t(2 * gamma);
  size_t off = 0;
  L.off_part = off;
  off += align256(sizeof(RowPart) * rows * size_t(L.nchunk));
  L.off_rowstat = off;
  off += align256(sizeof(RowStat) * rows);
  L.off_chunk_sum = off;
  off += align256(sizeof(double) * size_t(B) * size_t(gamma) * size_t(L.nchunk));
  L.total = off;
  return L;
}

struct AlphaArgs {
  const void* target;
  const void* draft;
  sv_dtype dtype;
  const float* temperature;
  int32_t B, gamma;
  int64_t V;
  float* out_alpha;
  int32_t* out_status;
  char* ws;
  bool vec;
};

// Workspace of the sampler: per (row, chunk) softmax partials.
struct SampleLayout {
  int64_t nchunk;
  size_t off_part, total;
};

inline SampleLayout sample_layout(int64_t rows, int64_t V) {
  SampleLayout L;
  L.nchunk = n_chunks(V);
  L.off_part = 0;
  L.total = align256(sizeof(RowPart) * size_t(rows) * size_t(L.nchunk));
  return L;
}

struct SampleArgs {
  const void* logits;
  sv_dtype dtype;
  const float* temperature;
  const float* uniforms;
  int32_t rows;
  int64_t V;
  int32_t* out_tokens;
  float* out_prob;
  int32_t* out_status;
  char* ws;
  bool vec;
};

// KV compaction geometry: kKvBlock-thread workgroups, each copying one tile of a row for one of
// kKvSlots groups of path slots; a tile is kKvVecPerThread words per thread, words of 16, 4 or 1
// bytes by alignment, so at least kKvMinTileBytes.  Measured on 256 chains of up to 8 rows of
// 128 KiB: 8 KiB tiles (two 16-byte words per thread) 49.6 us, 16 KiB tiles 56.2 us, 4 KiB tiles
// 67.2 us (the empty workgroups of slots past the accepted count then cost more than they save).
constexpr int kKvBlock = 256;
constexpr int kKvSlots = 8;
constexpr int kKvVecPerThread = 2;
constexpr int64_t kKvMinTileBytes = int64_t(kKvBlock) * kKvVecPerThread;

struct KvArgs {
  const void* src;
  void* dst;
  int64_t row_bytes;
  int32_t n, src_rows, dst_rows;
  const int32_t* path;
  int32_t path_len;
  const int32_t* num_accepted;
  const int32_t* dst_start;
  int32_t* out_status;
};

struct ChainArgs {
  const void* target;
  const void* draft;
  sv_dtype dtype;
  const int32_t* draft_tokens;
  const float* uniforms;
  const float* temperature;
  int32_t B, gamma;
  int64_t V;
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  float* out_p;
  float* out_q;
  int32_t* out_status;
  float* out_alpha;  // [B, gamma] acceptance rates, or NULL (plain verification)
  char* ws;
  bool vec;   // 16-byte vector-load path is legal
  bool lazy;  // early exit allowed: rows after the cut need not be read
};

struct TreeArgs {
  const void* logits;
  sv_dtype dtype;
  const int32_t* parents;
  const int32_t* node_tokens;
  int32_t n_trees, n_nodes;
  int64_t V;
  int32_t* out_path;
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  int32_t* out_node_argmax;
  int32_t* out_status;
  char* ws;
  bool vec;
};

struct GreedyArgs {
  const void* target;
  sv_dtype dtype;
  const int32_t* draft_tokens;
  int32_t B, gamma;
  int64_t V;
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  int32_t* out_argmax;
  int32_t* out_status;
  char* ws;
  bool vec;
};

// Launch the chain kernels on `stream`; returns hipSuccess or the launch error.
hipError_t launch_chain(const ChainArgs& a, hipStream_t stream);
hipError_t launch_tree(const TreeArgs& a, hipStream_t stream);
hipError_t launch_greedy(const GreedyArgs& a, hipStream_t stream);
hipError_t launch_alpha(const AlphaArgs& a, hipStream_t stream);
hipError_t launch_sample(const SampleArgs& a, hipStream_t stream);
hipError_t launch_kv_compact(const KvArgs& a, hipStream_t stream);

// The current device's copy of the static scratch array of the entry point that allocates
// nothing (its device address, looked up on the first call on each device).
hipError_t static_scratch(void** ptr);

// Streaming-read ceiling (measurement support): its geometry, the workgroups it launches for
// `bytes`, and the launch (one output word per workgroup).
constexpr int kProbeBlock = 1024;
constexpr int kProbeLoads = 8;                                  // 16-byte loads per lane
constexpr int64_t kProbeWave16 = int64_t(kWave) * kProbeLoads;  // 16-byte words per wave
inline int64_t read_probe_groups(int64_t bytes) {
  return ceil_div(bytes, int64_t(kProbeBlock / kWave) * kProbeWave16 * 16);
}
hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* out, hipStream_t s);

}  // namespace sv
