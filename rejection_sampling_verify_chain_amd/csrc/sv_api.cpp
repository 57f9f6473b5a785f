// C ABI of libspecverify: argument validation and dispatch to the kernel launchers.
//
// Nothing here allocates, synchronises or reads device memory: every check uses the
// arguments alone, and all work is enqueued on the caller's stream.

#include <stdint.h>

#include "sv_internal.h"
#include "specverify.h"

#define SV_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int vec_width(sv_dtype dtype) { return dtype == SV_F32 ? 4 : 8; }

bool valid_dtype(sv_dtype dtype) { return dtype == SV_F32 || dtype == SV_BF16; }


bool chain_shape_ok(int32_t B, int32_t gamma, int64_t V) {
  if (B < 1 || B > sv::kMaxBatch || gamma < 1 || gamma > sv::kMaxGamma) return false;
  if (V < 1 || V > int64_t(INT32_MAX)) return false;
  return sv::shape_grids_fit(B, 2 * gamma + 1, V);
}

bool tree_shape_ok(int32_t n_trees, int32_t n_nodes, int64_t V) {
  if (n_trees < 1 || n_trees > sv::kMaxBatch || n_nodes < 1 || n_nodes > sv::kMaxTreeNodes)
    return false;
  if (V < 1 || V > int64_t(INT32_MAX)) return false;
  return sv::shape_grids_fit(n_trees, n_nodes, V);
}

bool greedy_shape_ok(int32_t B, int32_t gamma, int64_t V) {
  if (B < 1 || B > sv::kMaxBatch || gamma < 1 || gamma > sv::kMaxGamma) return false;
  if (V < 1 || V > int64_t(INT32_MAX)) return false;
  return sv::shape_grids_fit(B, gamma + 1, V);
}

bool alpha_shape_ok(int32_t B, int32_t gamma, int64_t V) {
  if (B < 1 || B > sv::kMaxBatch || gamma < 1 || gamma > sv::kMaxGamma) return false;
  if (V < 1 || V > int64_t(INT32_MAX)) return false;
  return sv::shape_grids_fit(B, 2 * gamma, V);
}

bool sample_shape_ok(int32_t rows, int64_t V) {
  if (rows < 1 || rows > sv::kMaxBatch || V < 1 || V > int64_t(INT32_MAX)) return false;
  return sv::shape_grids_fit(rows, 1, V);
}

}  // namespace

SV_EXPORT const char* sv_version(void) { return "specverify 0.1.0 gfx950"; }

SV_EXPORT const char* sv_status_string(sv_status status) {
  switch (status) {
    case SV_OK: return "SV_OK";
    case SV_ERR_NULL: return "SV_ERR_NULL: a required pointer is NULL";
    case SV_ERR_SHAPE: return "SV_ERR_SHAPE: a size is out of range";
    case SV_ERR_DTYPE: return "SV_ERR_DTYPE: unknown logit dtype";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case SV_ERR_LAUNCH: return "SV_ERR_LAUNCH: kernel launch (or a runtime lookup) failed";
    case SV_ERR_SCRATCH:
      return "SV_ERR_SCRATCH: the call needs more than SV_NOALLOC_SCRATCH_BYTES of scratch";
  }
  return "unknown sv_status";
}

namespace {

sv_status verify_chain(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                       const int32_t* draft_tokens, const float* uniforms,
                       const float* temperature, int32_t B, int32_t gamma, int64_t V,
                       int32_t* out_tokens, int32_t* out_num_accepted, float* out_p, float* out_q,
                       int32_t* out_status, float* out_alpha, bool lazy, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !temperature ||
      !out_tokens || !out_num_accepted)
    return SV_ERR_NULL;
  if (!valid_dtype(dtype)) return SV_ERR_DTYPE;
  if (!chain_shape_ok(B, gamma, V)) return SV_ERR_SHAPE;
  const size_t need = sv::chain_layout(B, gamma, V, out_alpha != nullptr).total;
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return SV_ERR_WORKSPACE;

  sv::ChainArgs a;
  a.target = target_logits;
  a.draft = draft_logits;
  a.dtype = dtype;
  a.draft_tokens = draft_tokens;
  a.uniforms = uniforms;
  a.temperature = temperature;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.out_tokens = out_tokens;
  a.out_num_accepted = out_num_accepted;
  a.out_p = out_p;
  a.out_q = out_q;
  a.out_status = out_status;
  a.out_alpha = out_alpha;
  a.lazy = lazy;
  a.ws = static_cast<char*>(workspace);
  a.vec = aligned16(target_logits) && aligned16(draft_logits) && V % vec_width(dtype) == 0;
  return sv::launch_chain(a, stream) == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

}  // namespace

SV_EXPORT size_t sv_verify_chain_workspace_bytes(int32_t B, int32_t gamma, int64_t V,
                                                 sv_dtype dtype) {
  if (!valid_dtype(dtype) || !chain_shape_ok(B, gamma, V)) return 0;
  return sv::chain_layout(B, gamma, V).total;
}

SV_EXPORT sv_status sv_verify_chain(const void* target_logits, const void* draft_logits,
                                    sv_dtype dtype, const int32_t* draft_tokens,
                                    const float* uniforms, const float* temperature, int32_t B,
                                    int32_t gamma, int64_t V, int32_t* out_tokens,
                                    int32_t* out_num_accepted, float* out_p, float* out_q,
                                    int32_t* out_status, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  return verify_chain(target_logits, draft_logits, dtype, draft_tokens, uniforms, temperature, B,
                      gamma, V, out_tokens, out_num_accepted, out_p, out_q, out_status, nullptr,
                      false, workspace, workspace_bytes, stream);
}

SV_EXPORT sv_status sv_verify_chain_noalloc(const void* target_logits, const void* draft_logits,
                                            sv_dtype dtype, const int32_t* draft_tokens,
                                            const float* uniforms, const float* temperature,
                                            int32_t B, int32_t gamma, int64_t V,
                                            int32_t* out_tokens, int32_t* out_num_accepted,
                                            float* out_p, float* out_q, int32_t* out_status,
                                            hipStream_t stream) {
  if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !temperature ||
      !out_tokens || !out_num_accepted)
    return SV_ERR_NULL;
  if (!valid_dtype(dtype)) return SV_ERR_DTYPE;
  if (!chain_shape_ok(B, gamma, V)) return SV_ERR_SHAPE;
  const size_t need = sv::chain_layout(B, gamma, V).total;
  if (need > SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_SCRATCH;
  void* ws = nullptr;
  if (sv::static_scratch(&ws) != hipSuccess) return SV_ERR_LAUNCH;
  return verify_chain(target_logits, draft_logits, dtype, draft_tokens, uniforms, temperature, B,
                      gamma, V, out_tokens, out_num_accepted, out_p, out_q, out_status, nullptr,
                      false, ws, need, stream);
}

SV_EXPORT sv_status sv_verify_chain_lazy(const void* target_logits, const void* draft_logits,
                                         sv_dtype dtype, const int32_t* draft_tokens,
                                         const float* uniforms, const float* temperature,
                                         int32_t B, int32_t gamma, int64_t V, int32_t* out_tokens,
                                         int32_t* out_num_accepted, float* out_p, float* out_q,
                                         int32_t* out_status, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  return verify_chain(target_logits, draft_logits, dtype, draft_tokens, uniforms, temperature, B,
                      gamma, V, out_tokens, out_num_accepted, out_p, out_q, out_status, nullptr,
                      true, workspace, workspace_bytes, stream);
}

SV_EXPORT size_t sv_verify_chain_with_rates_workspace_bytes(int32_t B, int32_t gamma, int64_t V,
                                                            sv_dtype dtype) {
  if (!valid_dtype(dtype) || !chain_shape_ok(B, gamma, V)) return 0;
  return sv::chain_layout(B, gamma, V, true).total;
}

SV_EXPORT sv_status sv_verify_chain_with_rates(
    const void* target_logits, const void* draft_logits, sv_dtype dtype,
    const int32_t* draft_tokens, const float* uniforms, const float* temperature, int32_t B,
    int32_t gamma, int64_t V, int32_t* out_tokens, int32_t* out_num_accepted, float* out_p,
    float* out_q, int32_t* out_status, float* out_alpha, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  if (!out_alpha) return SV_ERR_NULL;
  return verify_chain(target_logits, draft_logits, dtype, draft_tokens, uniforms, temperature, B,
                      gamma, V, out_tokens, out_num_accepted, out_p, out_q, out_status, out_alpha,
                      false, workspace, workspace_bytes, stream);
}

SV_EXPORT size_t sv_verify_tree_workspace_bytes(int32_t n_trees, int32_t n_nodes, int64_t V,
                                                sv_dtype dtype) {
  if (!valid_dtype(dtype) || !tree_shape_ok(n_trees, n_nodes, V)) return 0;
  return sv::tree_layout(n_trees, n_nodes, V).total;
}

SV_EXPORT sv_status sv_verify_tree(const void* logits, sv_dtype dtype, const int32_t* parents,
                                   const int32_t* node_tokens, int32_t n_trees, int32_t n_nodes,
                                   int64_t V, int32_t* out_path, int32_t* out_tokens,
                                   int32_t* out_num_accepted, int32_t* out_node_argmax,
                                   int32_t* out_status, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  if (!logits || !parents || !node_tokens || !out_path || !out_tokens || !out_num_accepted)
    return SV_ERR_NULL;
  if (!valid_dtype(dtype)) return SV_ERR_DTYPE;
  if (!tree_shape_ok(n_trees, n_nodes, V)) return SV_ERR_SHAPE;
  const size_t need = sv::tree_layout(n_trees, n_nodes, V).total;
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return SV_ERR_WORKSPACE;

  sv::TreeArgs a;
  a.logits = logits;
  a.dtype = dtype;
  a.parents = parents;
  a.node_tokens = node_tokens;
  a.n_trees = n_trees;
  a.n_nodes = n_nodes;
  a.V = V;
  a.out_path = out_path;
  a.out_tokens = out_tokens;
  a.out_num_accepted = out_num_accepted;
  a.out_node_argmax = out_node_argmax;
  a.out_status = out_status;
  a.ws = static_cast<char*>(workspace);
  a.vec = aligned16(logits) && V % vec_width(dtype) == 0;
  return sv::launch_tree(a, stream) == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

SV_EXPORT size_t sv_verify_chain_greedy_workspace_bytes(int32_t B, int32_t gamma, int64_t V,
                                                        sv_dtype dtype) {
  if (!valid_dtype(dtype) || !greedy_shape_ok(B, gamma, V)) return 0;
  return sv::greedy_layout(B, gamma, V).total;
}

SV_EXPORT sv_status sv_verify_chain_greedy(const void* target_logits, sv_dtype dtype,
                                           const int32_t* draft_tokens, int32_t B, int32_t gamma,
                                           int64_t V, int32_t* out_tokens,
                                           int32_t* out_num_accepted, int32_t* out_argmax,
                                           int32_t* out_status, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  if (!target_logits || !draft_tokens || !out_tokens || !out_num_accepted) return SV_ERR_NULL;
  if (!valid_dtype(dtype)) return SV_ERR_DTYPE;
  if (!greedy_shape_ok(B, gamma, V)) return SV_ERR_SHAPE;
  const size_t need = sv::greedy_layout(B, gamma, V).total;
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return SV_ERR_WORKSPACE;

  sv::GreedyArgs a;
  a.target = target_logits;
  a.dtype = dtype;
  a.draft_tokens = draft_tokens;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.out_tokens = out_tokens;
  a.out_num_accepted = out_num_accepted;
  a.out_argmax = out_argmax;
  a.out_status = out_status;
  a.ws = static_cast<char*>(workspace);
  a.vec = aligned16(target_logits) && V % vec_width(dtype) == 0;
  return sv::launch_greedy(a, stream) == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

SV_EXPORT size_t sv_chain_acceptance_rates_workspace_bytes(int32_t B, int32_t gamma, int64_t V,
                                                           sv_dtype dtype) {
  if (!valid_dtype(dtype) || !alpha_shape_ok(B, gamma, V)) return 0;
  return sv::alpha_layout(B, gamma, V).total;
}

SV_EXPORT sv_status sv_chain_acceptance_rates(const void* target_logits, const void* draft_logits,
                                              sv_dtype dtype, const float* temperature,
                                              int32_t B, int32_t gamma, int64_t V,
                                              float* out_alpha, int32_t* out_status,
                                              void* workspace, size_t workspace_bytes,
                                              hipStream_t stream) {
  if (!target_logits || !draft_logits || !temperature || !out_alpha) return SV_ERR_NULL;
  if (!valid_dtype(dtype)) return SV_ERR_DTYPE;
  if (!alpha_shape_ok(B, gamma, V)) return SV_ERR_SHAPE;
  const size_t need = sv::alpha_layout(B, gamma, V).total;
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return SV_ERR_WORKSPACE;

  sv::AlphaArgs a;
  a.target = target_logits;
  a.draft = draft_logits;
  a.dtype = dtype;
  a.temperature = temperature;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.out_alpha = out_alpha;
  a.out_status = out_status;
  a.ws = static_cast<char*>(workspace);
  a.vec = aligned16(target_logits) && aligned16(draft_logits) && V % vec_width(dtype) == 0;
  return sv::launch_alpha(a, stream) == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

SV_EXPORT size_t sv_sample_workspace_bytes(int32_t rows, int64_t V, sv_dtype dtype) {
  if (!valid_dtype(dtype) || !sample_shape_ok(rows, V)) return 0;
  return sv::sample_layout(rows, V).total;
}

SV_EXPORT sv_status sv_sample(const void* logits, sv_dtype dtype, const float* temperature,
                              const float* uniforms, int32_t rows, int64_t V,
                              int32_t* out_tokens, float* out_prob, int32_t* out_status,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!logits || !temperature || !uniforms || !out_tokens) return SV_ERR_NULL;
  if (!valid_dtype(dtype)) return SV_ERR_DTYPE;
  if (!sample_shape_ok(rows, V)) return SV_ERR_SHAPE;
  const size_t need = sv::sample_layout(rows, V).total;
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return SV_ERR_WORKSPACE;

  sv::SampleArgs a;
  a.logits = logits;
  a.dtype = dtype;
  a.temperature = temperature;
  a.uniforms = uniforms;
  a.rows = rows;
  a.V = V;
  a.out_tokens = out_tokens;
  a.out_prob = out_prob;
  a.out_status = out_status;
  a.ws = static_cast<char*>(workspace);
  a.vec = aligned16(logits) && V % vec_width(dtype) == 0;
  return sv::launch_sample(a, stream) == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

SV_EXPORT sv_status sv_compact_accepted(const void* src, void* dst, int64_t row_bytes, int32_t n,
                                        int32_t src_rows, int32_t dst_rows, const int32_t* path,
                                        int32_t path_len, const int32_t* num_accepted,
                                        const int32_t* dst_start, int32_t* out_status,
                                        hipStream_t stream) {
  if (!src || !dst || !num_accepted || !dst_start) return SV_ERR_NULL;
  if (n < 1 || src_rows < 1 || dst_rows < 1 || row_bytes < 1) return SV_ERR_SHAPE;
  if (path && path_len < 1) return SV_ERR_SHAPE;
  if (row_bytes > (int64_t(1) << 40)) return SV_ERR_SHAPE;
  // Buffer sizes in bytes; a product past 2^63 describes no buffer.
  int64_t src_bytes = 0, dst_bytes = 0;
  if (__builtin_mul_overflow(int64_t(n) * src_rows, row_bytes, &src_bytes) ||
      __builtin_mul_overflow(int64_t(n) * dst_rows, row_bytes, &dst_bytes))
    return SV_ERR_SHAPE;
  // Grid: one workgroup per (sequence, path-slot group, tile of row bytes); it must stay below
  // 2^32 work-items (n * slots < 2^34 and tiles <= 2^30, so the product fits in 64 bits).
  const int64_t tiles = sv::ceil_div(row_bytes, sv::kKvMinTileBytes);
  if (!sv::work_items_fit(int64_t(n) * sv::kKvSlots * tiles, sv::kKvBlock)) return SV_ERR_SHAPE;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + uintptr_t(dst_bytes) && d0 < s0 + uintptr_t(src_bytes)) return SV_ERR_SHAPE;

  sv::KvArgs a;
  a.src = src;
  a.dst = dst;
  a.row_bytes = row_bytes;
  a.n = n;
  a.src_rows = src_rows;
  a.dst_rows = dst_rows;
  a.path = path;
  a.path_len = path_len;
  a.num_accepted = num_accepted;
  a.dst_start = dst_start;
  a.out_status = out_status;
  return sv::launch_kv_compact(a, stream) == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

// ---------------------------------------------------------------------- measurement support

SV_EXPORT size_t sv_read_probe_out_words(int64_t bytes) {
  if (bytes <= 0 || bytes % 16 != 0) return 0;
  const int64_t g = sv::read_probe_groups(bytes);
  return sv::work_items_fit(g, sv::kProbeBlock) ? size_t(g) : 0;
}

SV_EXPORT sv_status sv_read_probe(const void* src, int64_t bytes, uint32_t* out,
                                  hipStream_t stream) {
  if (!src || !out) return SV_ERR_NULL;
  if (sv_read_probe_out_words(bytes) == 0 || !aligned16(src)) return SV_ERR_SHAPE;
  return sv::launch_read_probe(src, bytes, out, stream) == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
