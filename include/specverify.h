/*
 * specverify — the target-side verify step of speculative sampling on MI355X (gfx950).
 *
 * C ABI.  Every array argument is a device pointer owned by the caller; the
 * library allocates nothing, never synchronises, and enqueues its kernels on
 * the caller's HIP stream.  Entry points are stateless and thread-safe; two
 * calls that share a workspace must not overlap in time (put them on one
 * stream, or give each its own workspace).
 *
 * Errors that the host can see from the arguments alone are returned as an
 * sv_status before anything is launched.  Errors that depend on the data
 * (a token out of range, a NaN logit, a bad temperature) cannot be seen
 * without reading device memory; they are reported per sequence or per tree
 * through the optional out_status array (SV_ROW_* bits) and the affected
 * entries take a defined, in-range fallback result.
 *
 * Sources of the operations (cited by page title and section):
 *  [SpS]  "論文解説: Speculative Sampling — ドラフトモデルによるLLMデコード高速化"
 *         (0h-n0.github.io explainer of arXiv:2302.01318): Step 2 (ステップ2),
 *         Step 3 (ステップ3) accept equation, modified rejection sampling
 *         (修正付き棄却サンプリング) equation, expected speedup (期待される高速化),
 *         the sequence diagram and the code sketch's speculative_decode
 *         (gamma = look-ahead, temperature applied to both models).
 *  [SpI]  SpecInfer article (abeam.tech, arXiv:2305.09781): basic idea
 *         (基本アイデア) and inference (推論方法) — token-tree verification.
 *  [SDE]  "投機的デコーディングとは？LLMの回答を高速化する仕組み"
 *         (ai-compass.weeybrid.co.jp): 候補の採用と棄却を具体例で見る — greedy verification.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of the logits.  bf16 values are 16-bit brain-float patterns;
 * both widen exactly to fp32 inside the kernels. */
typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

typedef enum {
  SV_OK = 0,
  SV_ERR_NULL = 1,      /* a required pointer is NULL                                  */
  SV_ERR_SHAPE = 2,     /* a size is out of range (see each entry point)               */
  SV_ERR_DTYPE = 3,     /* dtype is not an sv_dtype                                    */
  SV_ERR_WORKSPACE = 5, /* workspace is NULL or smaller than the *_workspace_bytes size */
  SV_ERR_LAUNCH = 6,    /* the HIP runtime refused a launch, or a lookup the call needs */
  SV_ERR_SCRATCH = 7    /* the call needs more than the library's static scratch holds  */
} sv_status;

/* Per-sequence / per-tree data-error bits written to out_status (0 = clean). */
enum {
  SV_ROW_TOKEN_RANGE = 1,     /* a draft token / tree node token is outside [0, V)            */
  SV_ROW_NONFINITE = 2,       /* a logit row holds NaN or +inf, or only -inf (chain); NaN (tree) */
  SV_ROW_RESIDUAL_ZERO = 4,   /* rejection with zero residual mass: drawn from p_k instead     */
  SV_ROW_BAD_TREE = 8,        /* parents[0] != -1 or parents[i] not in [0, i)                  */
  SV_ROW_BAD_TEMPERATURE = 16,/* temperature not finite and > 0                               */
  SV_ROW_BAD_UNIFORM = 32,    /* a uniform outside [0, 1)                                      */
  SV_ROW_BAD_INDEX = 64       /* KV compaction: a path entry, count or destination out of range */
};

/* Library version string, e.g. "specverify 0.1.0 gfx950". */
const char* sv_version(void);

/* Human-readable name of a status code (never NULL). */
const char* sv_status_string(sv_status status);

/* ------------------------------------------------------------------------------------------
 * Chain verification ([SpS] Step 2, Step 3, modified rejection sampling).
 *
 * For each sequence b with temperature T = temperature[b]:
 *   p_i = softmax(target_logits[b, i, :] / T)   i = 0..gamma   (row gamma = bonus position)
 *   q_i = softmax(draft_logits[b, i, :] / T)    i = 0..gamma-1
 *   draft token x_i = draft_tokens[b, i] is accepted while
 *       uniforms[b, i] < min(1, p_i(x_i) / q_i(x_i))          (strict; q = 0 < p counts as +inf,
 *                                                             p = q = 0 rejects)
 *   k = number of leading accepts (the cut at the first rejection, [SpS] Step 3).
 *   If k < gamma the replacement token is drawn from norm(max(0, p_k - q_k)); if that mass is
 *   zero it is drawn from p_k and SV_ROW_RESIDUAL_ZERO is set.  If k == gamma a bonus token is
 *   drawn from p_gamma.  Draws are by inverse CDF in token-id order with u = uniforms[b, gamma]:
 *       y = min{ x : sum_{t<=x} w(t) > u * sum_t w(t) }.
 *   out_tokens[b, :] = [x_0 .. x_{k-1}, y, -1 ...]; out_num_accepted[b] = k (k+1 tokens emitted).
 *
 * Arguments (all device pointers, caller-owned, contiguous row-major):
 *   target_logits  [B, gamma+1, V] of dtype; target row i scores draft token i.
 *   draft_logits   [B, gamma, V]   of dtype.
 *   draft_tokens   int32 [B, gamma].
 *   uniforms       fp32 [B, gamma+1]; columns 0..gamma-1 drive the accept tests, column gamma
 *                  the draw.  The caller draws them (the library holds no random state).
 *   temperature    fp32 [B].
 *   B in [1, 2^22 - 1], gamma in [1, 64], V in [1, 2^31 - 1], and
 *   B * (2*gamma + 1) * ceil(V / 2048) <= 2^26 - 16: every launch stays below 2^32 work-items
 *   (one wavefront per 2048 logits, one 1024-thread workgroup per sequence); else SV_ERR_SHAPE.
 *   out_tokens        int32 [B, gamma+1]  (required)
 *   out_num_accepted  int32 [B]           (required)
 *   out_p, out_q      fp32 [B, gamma]: p_i(x_i), q_i(x_i) for every i < gamma (optional, NULL)
 *   out_status        int32 [B]: SV_ROW_* bits (optional, NULL)
 *   workspace         device scratch of at least sv_verify_chain_workspace_bytes(B, gamma, V,
 *                     dtype) bytes, 256-byte aligned; no initialisation needed; contents are
 *                     undefined after the call.
 * Sequences with SV_ROW_TOKEN_RANGE, SV_ROW_NONFINITE, SV_ROW_BAD_TEMPERATURE or
 * SV_ROW_BAD_UNIFORM take the fallback result k = 0, out_tokens = [0, -1, ...]; their out_p /
 * out_q are unspecified.
 * Any base pointer alignment is accepted; 16-byte-aligned logits with V a multiple of 4 (fp32)
 * or 8 (bf16) take the vector-load path.
 * Execution (vector-load path; all give bit-identical results): one launch with one workgroup
 * per sequence when a sequence has at most 256 KiB of logits and B <= 256, or when 192 <= B <=
 * 256; else a sweep across the chip followed by one workgroup per sequence when B <= 512 and a
 * sequence's residual re-read (2 * V elements) is at most 256 KiB; else four launches.  Rows
 * that are not 16-byte aligned always take four launches.  The environment variable
 * SPECVERIFY_CHAIN_PATH=fused, =finish or =split, read on every call, forces one of them where
 * the sequence's partials fit the one-workgroup form's 32 KiB LDS budget (testing and
 * measurement).
 * ---------------------------------------------------------------------------------------- */
size_t sv_verify_chain_workspace_bytes(int32_t B, int32_t gamma, int64_t V, sv_dtype dtype);

sv_status sv_verify_chain(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                          const int32_t* draft_tokens, const float* uniforms,
                          const float* temperature, int32_t B, int32_t gamma, int64_t V,
                          int32_t* out_tokens, int32_t* out_num_accepted, float* out_p,
                          float* out_q, int32_t* out_status, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Chain verification that allocates nothing, for callers that cannot allocate device memory
 * during the call or provide a workspace: code under HIP graph capture, tight serving loops,
 * and harnesses that forbid allocation.
 *
 * Exactly sv_verify_chain (same arguments apart from the workspace, same kernels, the same
 * outputs bit for bit), with its workspace taken from a static device array of
 * SV_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the process
 * ends.  The call allocates nothing and frees nothing.  Its first call on a device, with that
 * device current, looks up that device's copy of the array (an error there returns
 * SV_ERR_LAUNCH).  A call whose workspace (sv_verify_chain_workspace_bytes(B, gamma, V, dtype))
 * exceeds SV_NOALLOC_SCRATCH_BYTES returns SV_ERR_SCRATCH before launching anything; use
 * sv_verify_chain with a caller workspace for such shapes.  All calls on one GPU share the
 * array: calls that overlap in time on one GPU (two streams, or two host threads) race and
 * give undefined results; calls in order on one stream are safe.  Nothing in the array needs
 * clearing between calls.  Other errors as sv_verify_chain.
 * ---------------------------------------------------------------------------------------- */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

sv_status sv_verify_chain_noalloc(const void* target_logits, const void* draft_logits,
                                  sv_dtype dtype, const int32_t* draft_tokens,
                                  const float* uniforms, const float* temperature, int32_t B,
                                  int32_t gamma, int64_t V, int32_t* out_tokens,
                                  int32_t* out_num_accepted, float* out_p, float* out_q,
                                  int32_t* out_status, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Chain verification with early exit ([SpS] Step 3: the tests run in order and stop at the first
 * rejection, so the rows of later positions are never needed).
 *
 * Same arguments, workspace size (sv_verify_chain_workspace_bytes) and errors as
 * sv_verify_chain.  For inputs whose logit rows are all finite (no NaN, no +inf, not all -inf)
 * out_tokens, out_num_accepted and out_status equal sv_verify_chain's bit for bit, and so do
 * out_p / out_q at positions i <= k; after the cut they are NaN where the row was not read and
 * sv_verify_chain's values elsewhere.
 * Rows after the cut may not be read: a non-finite value there may or may not set
 * SV_ROW_NONFINITE and the fallback.  Batches with enough rows take the positions in order,
 * reading target and draft row i only once position i is reached (and target row gamma only if
 * every draft is accepted): for wide rows (a target and draft row of 512 KiB or more together,
 * or 256 KiB from 384 sequences on, or a first row pair of 48 MiB or more over the batch below
 * 256 sequences) two launches per position across the whole chip, the last of them taking
 * every remaining row, then the residual and draw kernels; from 256 sequences on with narrower
 * rows, one launch with one workgroup per sequence.  Other batches (and every batch below 128
 * sequences) run as sv_verify_chain.
 * SPECVERIFY_CHAIN_PATH=staged or =lazy, read on every call, forces the one-launch-per-position
 * form or the one-workgroup form at any batch size (testing and measurement; the one-workgroup
 * form needs the row pair's partials to fit 32 KiB of LDS).
 * ---------------------------------------------------------------------------------------- */
sv_status sv_verify_chain_lazy(const void* target_logits, const void* draft_logits,
                               sv_dtype dtype, const int32_t* draft_tokens, const float* uniforms,
                               const float* temperature, int32_t B, int32_t gamma, int64_t V,
                               int32_t* out_tokens, int32_t* out_num_accepted, float* out_p,
                               float* out_q, int32_t* out_status, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Chain verification with per-position acceptance rates ([SpS] Step 3 and expected speedup:
 * the accept probability alpha, watched in monitoring).
 *
 * Exactly sv_verify_chain (same arguments, same outputs, bit for bit), plus
 *   out_alpha  fp32 [B, gamma] (required): alpha_i = sum_x min(p_i(x), q_i(x)), the probability
 *              that draft token i is accepted when drawn from q_i, for every position i < gamma
 *              (NaN where target row i or draft row i has no softmax).  The values equal those of
 *              sv_chain_acceptance_rates on the same inputs bit for bit.
 * The rates reuse the verification's sweep and row statistics, so they cost one more pass over
 * the gamma target and gamma draft rows.  This call always takes the four-launch path, followed
 * by two more launches.  workspace: at least sv_verify_chain_with_rates_workspace_bytes(B,
 * gamma, V, dtype) bytes, 256-byte aligned.  Errors as sv_verify_chain; a NULL out_alpha is
 * SV_ERR_NULL.
 * ---------------------------------------------------------------------------------------- */
size_t sv_verify_chain_with_rates_workspace_bytes(int32_t B, int32_t gamma, int64_t V,
                                                  sv_dtype dtype);

sv_status sv_verify_chain_with_rates(const void* target_logits, const void* draft_logits,
                                     sv_dtype dtype, const int32_t* draft_tokens,
                                     const float* uniforms, const float* temperature, int32_t B,
                                     int32_t gamma, int64_t V, int32_t* out_tokens,
                                     int32_t* out_num_accepted, float* out_p, float* out_q,
                                     int32_t* out_status, float* out_alpha, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Greedy token-tree verification ([SpI] basic idea, inference).
 *
 * For each tree t: g[u] = argmax_x logits[t, u, x] for every node u (lowest x on ties, -0 == +0,
 * NaN never the maximum).  Starting at the root u = 0, repeatedly move to the child c of u
 * (lowest node id among children) with node_tokens[t, c] == g[u]; stop when there is none.
 *   out_path[t, :]   = [0, c_1, .., c_k, -1 ...]          node ids of the accepted path
 *   out_tokens[t, :] = [tok(c_1) .. tok(c_k), g[c_k], -1 ...]   accepted tokens + bonus argmax
 *   out_num_accepted[t] = k
 *
 * Arguments (device pointers, caller-owned):
 *   logits       [n_trees, n_nodes, V] of dtype; row u scores the children of node u.
 *   parents      int32 [n_trees, n_nodes]; parents[t,0] = -1 and 0 <= parents[t,i] < i.
 *   node_tokens  int32 [n_trees, n_nodes]; node 0 holds the last committed token (not emitted).
 *   n_trees in [1, 2^22 - 1], n_nodes in [1, 4096], V in [1, 2^31 - 1], and
 *   n_trees * n_nodes * ceil(V / 2048) <= 2^26 - 16 (launches below 2^32 work-items).
 *   out_path, out_tokens  int32 [n_trees, n_nodes] (required)
 *   out_num_accepted      int32 [n_trees]          (required)
 *   out_node_argmax       int32 [n_trees, n_nodes] g[u] (optional, NULL)
 *   out_status            int32 [n_trees] SV_ROW_* bits (optional, NULL)
 *   workspace             at least sv_verify_tree_workspace_bytes(...) bytes, 256-byte aligned.
 * A tree with SV_ROW_BAD_TREE or SV_ROW_TOKEN_RANGE takes the fallback result: path [0],
 * tokens [g[0]], k = 0.  NaN logits set SV_ROW_NONFINITE; NaN entries are skipped by the argmax
 * (a row of only NaN gives 0) and the walk proceeds.
 * ---------------------------------------------------------------------------------------- */
size_t sv_verify_tree_workspace_bytes(int32_t n_trees, int32_t n_nodes, int64_t V,
                                      sv_dtype dtype);

sv_status sv_verify_tree(const void* logits, sv_dtype dtype, const int32_t* parents,
                         const int32_t* node_tokens, int32_t n_trees, int32_t n_nodes, int64_t V,
                         int32_t* out_path, int32_t* out_tokens, int32_t* out_num_accepted,
                         int32_t* out_node_argmax, int32_t* out_status, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Greedy chain verification ("投機的デコーディングとは？LLMの回答を高速化する仕組み",
 * ai-compass.weeybrid.co.jp, section 候補の採用と棄却を具体例で見る: candidates are kept while
 * they equal the target's own choice; the first that differs is replaced by that choice).  The
 * zero-temperature form of chain verification: no draft logits, no random numbers.
 *
 * For each sequence b: g_i = argmax_x target_logits[b, i, x] for i = 0..gamma (lowest x on
 * ties, -0 == +0, NaN never the maximum); k = number of leading i < gamma with
 * draft_tokens[b, i] == g_i; out_tokens[b, :] = [x_0 .. x_{k-1}, g_k, -1 ...];
 * out_num_accepted[b] = k (k+1 tokens emitted).
 *
 * Arguments (device pointers, caller-owned, contiguous row-major):
 *   target_logits  [B, gamma+1, V] of dtype; target row i scores draft token i, row gamma is
 *                  the position after the last draft token.
 *   draft_tokens   int32 [B, gamma].
 *   B in [1, 2^22 - 1], gamma in [1, 64], V in [1, 2^31 - 1], and
 *   B * (gamma + 1) * ceil(V / 2048) <= 2^26 - 16 (launches below 2^32 work-items).
 *   out_tokens        int32 [B, gamma+1]  (required)
 *   out_num_accepted  int32 [B]           (required)
 *   out_argmax        int32 [B, gamma+1]: g_i (optional, NULL)
 *   out_status        int32 [B]: SV_ROW_* bits (optional, NULL)
 *   workspace         at least sv_verify_chain_greedy_workspace_bytes(B, gamma, V, dtype)
 *                     bytes, 256-byte aligned; no initialisation needed.
 * A draft token outside [0, V) sets SV_ROW_TOKEN_RANGE and the sequence takes the fallback
 * result k = 0, out_tokens = [g_0, -1, ...].  A NaN logit sets SV_ROW_NONFINITE; NaN entries
 * are skipped by the argmax (a row of only NaN gives 0) and the comparison proceeds.
 * ---------------------------------------------------------------------------------------- */
size_t sv_verify_chain_greedy_workspace_bytes(int32_t B, int32_t gamma, int64_t V,
                                              sv_dtype dtype);

sv_status sv_verify_chain_greedy(const void* target_logits, sv_dtype dtype,
                                 const int32_t* draft_tokens, int32_t B, int32_t gamma, int64_t V,
                                 int32_t* out_tokens, int32_t* out_num_accepted,
                                 int32_t* out_argmax, int32_t* out_status, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Per-position acceptance rates ([SpS] Step 3 accept probability, expected-speedup alpha, and
 * the deployment section's monitoring of alpha): for each sequence b and position i < gamma,
 *   alpha_i = sum_x q_i(x) min(1, p_i(x) / q_i(x)) = sum_x min(p_i(x), q_i(x)),
 * the probability that a token drafted from q_i is accepted, with p_i, q_i the temperature
 * softmaxes of target row i and draft row i as in sv_verify_chain.  Telemetry: it reads every
 * target and draft row twice (softmax statistics, then the overlap), independently of any verify
 * call.
 *
 * Arguments (device pointers, caller-owned, contiguous row-major):
 *   target_logits  [B, gamma+1, V] of dtype (the layout of sv_verify_chain; row gamma is not read).
 *   draft_logits   [B, gamma, V]   of dtype.
 *   temperature    fp32 [B].
 *   B in [1, 2^22 - 1], gamma in [1, 64], V in [1, 2^31 - 1], and
 *   B * 2*gamma * ceil(V / 2048) <= 2^26 - 16 (launches below 2^32 work-items).
 *   out_alpha      fp32 [B, gamma]  (required)
 *   out_status     int32 [B, gamma]: SV_ROW_* bits of each position (optional, NULL)
 *   workspace      at least sv_chain_acceptance_rates_workspace_bytes(B, gamma, V, dtype)
 *                  bytes, 256-byte aligned; no initialisation needed.
 * A position whose target or draft row defines no softmax (NaN, +inf, only -inf) gets NaN and
 * SV_ROW_NONFINITE; a temperature that is not finite and positive is replaced by 1 and sets
 * SV_ROW_BAD_TEMPERATURE on every position of the sequence.
 * ---------------------------------------------------------------------------------------- */
size_t sv_chain_acceptance_rates_workspace_bytes(int32_t B, int32_t gamma, int64_t V,
                                                 sv_dtype dtype);

sv_status sv_chain_acceptance_rates(const void* target_logits, const void* draft_logits,
                                    sv_dtype dtype, const float* temperature, int32_t B,
                                    int32_t gamma, int64_t V, float* out_alpha,
                                    int32_t* out_status, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Draft-side sampler ([SpS] Step 1 and the code sketch's draft loop: each draft token is drawn
 * from the softmax of the draft's logits divided by the temperature).
 *
 * For each row r: p = softmax(logits[r, :] / temperature[r]) and
 *   out_tokens[r] = y = min{ x : sum_{t<=x} p(t) > uniforms[r] * sum_t p(t) }
 * (inverse CDF in token-id order, the draw sv_verify_chain uses for its bonus token; a token of
 * probability zero is never drawn); out_prob[r] = p(y).
 *
 * Arguments (device pointers, caller-owned):
 *   logits       [rows, V] of dtype, contiguous rows.
 *   temperature  fp32 [rows], finite and > 0.
 *   uniforms     fp32 [rows] in [0, 1), drawn by the caller.
 *   rows in [1, 2^22 - 1], V in [1, 2^31 - 1], rows * ceil(V / 2048) <= 2^26 - 16 (launches
 *   below 2^32 work-items).
 *   out_tokens   int32 [rows] (required)
 *   out_prob     fp32 [rows]: p(y) (optional, NULL)
 *   out_status   int32 [rows]: SV_ROW_* bits (optional, NULL)
 *   workspace    at least sv_sample_workspace_bytes(rows, V, dtype) bytes, 256-byte aligned.
 * A row with SV_ROW_NONFINITE, SV_ROW_BAD_TEMPERATURE or SV_ROW_BAD_UNIFORM takes token 0 and
 * out_prob NaN.
 * ---------------------------------------------------------------------------------------- */
size_t sv_sample_workspace_bytes(int32_t rows, int64_t V, sv_dtype dtype);

sv_status sv_sample(const void* logits, sv_dtype dtype, const float* temperature,
                    const float* uniforms, int32_t rows, int64_t V, int32_t* out_tokens,
                    float* out_prob, int32_t* out_status, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Accepted-path KV compaction ([SpS] implementation notes, KV cache management: the cache
 * entries of rejected tokens are rolled back; [SpI] inference: the verified run is appended to
 * the sequence).
 *
 * The verification pass computed one KV row per speculated position, including the position
 * that feeds the first draft (a chain's last committed token, a tree's root): row u of sequence
 * b's block belongs to node u (chain position u).  For each sequence b with k = num_accepted[b]:
 *   for j = 0..k:  dst row (dst_start[b] + j) of sequence b  <-  src row path[b][j] of sequence b
 * with path[b][j] = j when path is NULL (a chain).  Rows of rejected nodes are not read.  The
 * path and count are those sv_verify_tree (out_path, out_num_accepted) or sv_verify_chain /
 * sv_verify_chain_greedy (out_num_accepted, path NULL) return.
 *
 * Arguments (device pointers, caller-owned):
 *   src           bytes [n, src_rows, row_bytes]: each sequence's speculative KV block.
 *   dst           bytes [n, dst_rows, row_bytes]: each sequence's cache; must not overlap src.
 *   row_bytes     bytes per KV row (all layers, keys and values, of one position), in
 *                 [1, 2^40]; n * 8 * ceil(row_bytes / 512) * 256 below 2^32 (the launch's
 *                 work-items) and n * max(src_rows, dst_rows) * row_bytes below 2^63.
 *   path          int32 [n, path_len] node ids (-1 padded), or NULL for chains.
 *   num_accepted  int32 [n]; dst_start int32 [n]: first destination row of each sequence.
 *   out_status    int32 [n]: SV_ROW_BAD_INDEX or 0 (optional, NULL).
 * A sequence with k outside [0, path_len - 1] (src_rows - 1 without a path), a path entry outside
 * [0, src_rows), or dst_start[b] + k + 1 > dst_rows sets SV_ROW_BAD_INDEX and copies nothing.
 * Overlapping src and dst ranges return SV_ERR_SHAPE.  No workspace.  Rows use 16-byte accesses
 * when src, dst and row_bytes are multiples of 16.
 * ---------------------------------------------------------------------------------------- */
sv_status sv_compact_accepted(const void* src, void* dst, int64_t row_bytes, int32_t n,
                              int32_t src_rows, int32_t dst_rows, const int32_t* path,
                              int32_t path_len, const int32_t* num_accepted,
                              const int32_t* dst_start, int32_t* out_status, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Kernel timing (measurement support; not part of the verify step).
 *
 * sv_trace_start(capacity): from now on, each kernel the library launches (up to `capacity`
 *   launches in total) is given two HIP events that the launch stamps with the start and end
 *   of that kernel's execution on its stream (hipExtLaunchKernel's events).  Creates
 *   2*capacity HIP events (host-side objects; no device memory).  Returns 0, or -1 if event
 *   creation failed.  Calling it again discards earlier records.
 * sv_trace_stop(): stops recording; returns the number of launches recorded.
 * sv_trace_kernels(): stops recording, waits for the recorded events, groups the launches by
 *   kernel name and returns the number of distinct names (-1 on a HIP error).
 * sv_trace_get(i, ...): name, launch count and total / min / max event-to-event milliseconds
 *   of the i-th name from the last sv_trace_kernels(); returns 0, or -1 for a bad index.
 * Not thread-safe with respect to concurrent verify calls on other threads.
 * ---------------------------------------------------------------------------------------- */
int sv_trace_start(int capacity);
int sv_trace_stop(void);
int sv_trace_kernels(void);
int sv_trace_get(int index, char* name, size_t name_len, int* launches, double* total_ms,
                 double* min_ms, double* max_ms);

/* ------------------------------------------------------------------------------------------
 * Streaming-read ceiling (measurement support; not part of the verify step).
 *
 * sv_read_probe(src, bytes, out, stream): reads the `bytes` bytes at device address src once,
 *   the way the streaming kernels read logits (one 8 KiB piece per wave as 16-byte nontemporal
 *   loads, 1024-thread workgroups), and writes the XOR of the 32-bit words each workgroup read to
 *   out (device, uint32 [sv_read_probe_out_words(bytes)], caller-owned), so that no load is
 *   dropped.  Its kernel time (traced as "read_probe") is the rate of a plain read of that size.
 *   Returns SV_ERR_NULL for a NULL pointer, SV_ERR_SHAPE when bytes is not a positive multiple
 *   of 16 or src is not 16-byte aligned, SV_ERR_LAUNCH if the launch fails, else SV_OK.
 * sv_read_probe_out_words(bytes): output words for that size (0 when the size is invalid).
 * ---------------------------------------------------------------------------------------- */
size_t sv_read_probe_out_words(int64_t bytes);
sv_status sv_read_probe(const void* src, int64_t bytes, uint32_t* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
