// Host-only check of the C ABI's validation and of the layout and grid arithmetic the kernels
// rely on, built with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitized.py).
//
// It links the library's argument-validation layer (sv_api.cpp) against the stub launchers
// below instead of the HIP kernels.  Every call that passes validation reaches a stub, which
// checks what the kernels assume about it:
//   * the workspace layout: every region 256-byte aligned, in order, large enough for its
//     entries and inside the workspace the call validated;
//   * every grid: each launch's work-items (workgroups x threads: one wave per chunk in
//     workgroups of up to 16 waves, or one workgroup of up to 1024 threads per sequence, tree
//     or row) below 2^32, the dispatch's 32-bit grid size;
//   * the largest element index a kernel forms (the last logit of the last row, the last
//     partial, the last KV byte) fits in 64 bits.
// main() drives every validation path of every entry point, the shape limits and just past
// them, and a sweep of shapes up to B = 2^22 - 1, gamma = 64, V = 2^31 - 1 and n_nodes = 4096.
// No device memory is touched: the pointers are fake addresses that are never dereferenced.

#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "specverify.h"
#include "sv_internal.h"

namespace {

int g_fail = 0;
long g_checks = 0;
long g_launches = 0;

#define CHECK(c)                                                                 \
  do {                                                                           \
    ++g_checks;                                                                  \
    if (!(c)) {                                                                  \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c);      \
      ++g_fail;                                                                  \
    }                                                                            \
  } while (0)

// CHECK with the shape printed on failure.
#define CHECK_AT(c, fmt, ...)                                                    \
  do {                                                                           \
    ++g_checks;                                                                  \
    if (!(c)) {                                                                  \
      fprintf(stderr, "%s:%d: check failed: %s at " fmt "\n", __FILE__, __LINE__, #c, \
              __VA_ARGS__);                                                      \
      ++g_fail;                                                                  \
    }                                                                            \
  } while (0)

// a * b, recording a failure if it leaves int64.
int64_t mul(int64_t a, int64_t b) {
  int64_t r = 0;
  const bool over = __builtin_mul_overflow(a, b, &r);
  CHECK(!over);
  return over ? INT64_MAX : r;
}

// `groups` workgroups of `threads` threads: a launchable grid.
void grid_ok(int64_t groups, int64_t threads) {
  CHECK(groups >= 1 && mul(groups, threads) <= sv::kMaxWorkItems);
}

// A launch with one wave per unit, in workgroups of 4 or 16 waves (the launchers' sizes).
void wave_grid_ok(int64_t units) {
  for (int64_t w : {4, 16}) grid_ok(sv::wave_groups(units, w), w * sv::kWave);
}

struct Region {
  size_t off, bytes;
};

void layout_ok(std::initializer_list<Region> regions, size_t total, const char* ws,
               size_t ws_bytes) {
  size_t end = 0;
  for (const Region& r : regions) {
    CHECK(r.off % 256 == 0);
    CHECK(r.off >= end);
    end = r.off + r.bytes;
  }
  CHECK(end <= total);
  CHECK(total % 256 == 0);
  CHECK(ws != nullptr && reinterpret_cast<uintptr_t>(ws) % 256 == 0);
  CHECK(total <= ws_bytes);
}

char* const kFake = reinterpret_cast<char*>(uintptr_t(1) << 20);  // 256-byte aligned, never read
size_t g_ws_bytes = 0;  // the workspace size the current call passed

}  // namespace

namespace sv {

hipError_t launch_chain(const ChainArgs& a, hipStream_t) {
  ++g_launches;
  CHECK(a.target && a.draft && a.draft_tokens && a.uniforms && a.temperature);
  CHECK(a.out_tokens && a.out_num_accepted);
  CHECK(a.B >= 1 && a.B <= kMaxBatch && a.gamma >= 1 && a.gamma <= kMaxGamma && a.V >= 1);
  const bool rates = a.out_alpha != nullptr;
  const ChainLayout L = chain_layout(a.B, a.gamma, a.V, rates);
  const int64_t rows = mul(a.B, 2 * a.gamma + 1);
  const int64_t units = mul(rows, L.nchunk);
  layout_ok({{L.off_part, size_t(mul(units, sizeof(RowPart)))},
             {L.off_rowstat, size_t(mul(rows, sizeof(RowStat)))},
             {L.off_seq, size_t(mul(a.B, sizeof(SeqDecision)))},
             {L.off_wres, size_t(mul(mul(a.B, L.nchunk), sizeof(double)))},
             {L.off_live, size_t(mul(mul(a.B, kStageLists) + kStageCountPad, sizeof(int32_t)))},
             {L.off_hstat, size_t(mul(a.B, sizeof(int32_t)))},
             {L.off_reached, size_t(mul(a.B, sizeof(int32_t)))},
             {L.off_lz, size_t(mul(mul(a.B, a.gamma), 2 * sizeof(float)))},
             {L.off_alpha_sum,
              rates ? size_t(mul(mul(mul(a.B, a.gamma), L.nchunk), sizeof(double))) : 0}},
            L.total, a.ws, g_ws_bytes);
  wave_grid_ok(units);                         // sweep: one wave per (row, chunk)
  wave_grid_ok(mul(a.B, L.nchunk));            // residual: one wave per (sequence, chunk)
  if (rates) wave_grid_ok(mul(mul(a.B, a.gamma), L.nchunk));  // overlap sums
  grid_ok(a.B, 1024);                          // one workgroup per sequence
  // Largest element indexes: the last logit of the target and draft blocks, the last partial.
  mul(mul(a.B, a.gamma + 1), a.V);
  mul(mul(a.B, a.gamma), a.V);
  CHECK(units - 1 < INT64_MAX);
  return hipSuccess;
}

hipError_t launch_tree(const TreeArgs& a, hipStream_t) {
  ++g_launches;
  CHECK(a.logits && a.parents && a.node_tokens && a.out_path && a.out_tokens &&
        a.out_num_accepted);
  CHECK(a.n_nodes >= 1 && a.n_nodes <= kMaxTreeNodes && a.n_trees >= 1 && a.V >= 1);
  const TreeLayout L = tree_layout(a.n_trees, a.n_nodes, a.V);
  const int64_t units = mul(mul(a.n_trees, a.n_nodes), L.nchunk);
  layout_ok({{L.off_part, size_t(mul(units, sizeof(ArgPart)))}}, L.total, a.ws, g_ws_bytes);
  wave_grid_ok(units);
  grid_ok(a.n_trees, 1024);
  // The walk's dynamic LDS: argmax, token and next child of every node.
  CHECK(3 * sizeof(int32_t) * size_t(a.n_nodes) <= 64 * 1024);
  mul(mul(a.n_trees, a.n_nodes), a.V);
  return hipSuccess;
}

hipError_t launch_greedy(const GreedyArgs& a, hipStream_t) {
  ++g_launches;
  CHECK(a.target && a.draft_tokens && a.out_tokens && a.out_num_accepted);
  const GreedyLayout L = greedy_layout(a.B, a.gamma, a.V);
  const int64_t units = mul(mul(a.B, a.gamma + 1), L.nchunk);
  layout_ok({{L.off_part, size_t(mul(units, sizeof(ArgPart)))}}, L.total, a.ws, g_ws_bytes);
  wave_grid_ok(units);
  grid_ok(a.B, 1024);
  mul(mul(a.B, a.gamma + 1), a.V);
  return hipSuccess;
}

hipError_t launch_alpha(const AlphaArgs& a, hipStream_t) {
  ++g_launches;
  CHECK(a.target && a.draft && a.temperature && a.out_alpha);
  const AlphaLayout L = alpha_layout(a.B, a.gamma, a.V);
  const int64_t rows = mul(a.B, 2 * a.gamma);
  layout_ok({{L.off_part, size_t(mul(mul(rows, L.nchunk), sizeof(RowPart)))},
             {L.off_rowstat, size_t(mul(rows, sizeof(RowStat)))},
             {L.off_chunk_sum, size_t(mul(mul(mul(a.B, a.gamma), L.nchunk), sizeof(double)))}},
            L.total, a.ws, g_ws_bytes);
  wave_grid_ok(mul(rows, L.nchunk));
  wave_grid_ok(rows);
  mul(mul(a.B, a.gamma + 1), a.V);
  return hipSuccess;
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t) {
  ++g_launches;
  CHECK(a.logits && a.temperature && a.uniforms && a.out_tokens);
  const SampleLayout L = sample_layout(a.rows, a.V);
  const int64_t units = mul(a.rows, L.nchunk);
  layout_ok({{L.off_part, size_t(mul(units, sizeof(RowPart)))}}, L.total, a.ws, g_ws_bytes);
  wave_grid_ok(units);
  grid_ok(a.rows, sv::kWave);
  mul(a.rows, a.V);
  return hipSuccess;
}

hipError_t launch_kv_compact(const KvArgs& a, hipStream_t) {
  ++g_launches;
  CHECK(a.src && a.dst && a.num_accepted && a.dst_start);
  CHECK(a.row_bytes >= 1 && a.row_bytes <= (int64_t(1) << 40));
  for (int64_t word : {1, 4, 16})  // the tile of each copy form
    grid_ok(mul(mul(a.n, kKvSlots), ceil_div(a.row_bytes, kKvMinTileBytes * word)), kKvBlock);
  // The last byte of the last source and destination row.
  mul(mul(a.n, a.src_rows), a.row_bytes);
  mul(mul(a.n, a.dst_rows), a.row_bytes);
  return hipSuccess;
}

hipError_t static_scratch(void** ptr) {
  *ptr = kFake;
  return hipSuccess;
}

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* out, hipStream_t) {
  ++g_launches;
  CHECK(src && out && bytes > 0 && bytes % 16 == 0);
  grid_ok(read_probe_groups(bytes), kProbeBlock);
  return hipSuccess;
}

}  // namespace sv

namespace {

const void* F = kFake;
int32_t* FI = reinterpret_cast<int32_t*>(kFake);
float* FF = reinterpret_cast<float*>(kFake);
const int32_t* CI = FI;
const float* CF = FF;

// Calls sv_verify_chain with a workspace of exactly its size (or `ws_bytes`), and checks the
// status; a launch happens exactly when the status is SV_OK.
void chain(int32_t B, int32_t gamma, int64_t V, sv_status want, sv_dtype dt = SV_BF16,
           size_t ws_bytes = 0, void* ws = kFake) {
  const size_t need = sv_verify_chain_workspace_bytes(B, gamma, V, dt);
  g_ws_bytes = ws_bytes ? ws_bytes : need;
  const long before = g_launches;
  const sv_status st = sv_verify_chain(F, F, dt, CI, CF, CF, B, gamma, V, FI, FI, FF, FF, FI, ws,
                                       g_ws_bytes, nullptr);
  CHECK_AT(st == want, "chain B=%d gamma=%d V=%lld: status %d, want %d", B, gamma, (long long)V,
           int(st), int(want));
  CHECK((g_launches > before) == (st == SV_OK));
  if (want == SV_OK) {
    CHECK(sv_verify_chain_lazy(F, F, dt, CI, CF, CF, B, gamma, V, FI, FI, nullptr, nullptr,
                               nullptr, ws, g_ws_bytes, nullptr) == SV_OK);
    const size_t rneed = sv_verify_chain_with_rates_workspace_bytes(B, gamma, V, dt);
    CHECK(rneed >= need);
    g_ws_bytes = rneed;
    CHECK(sv_verify_chain_with_rates(F, F, dt, CI, CF, CF, B, gamma, V, FI, FI, FF, FF, FI, FF,
                                     ws, rneed, nullptr) == SV_OK);
    CHECK(sv_verify_chain_with_rates(F, F, dt, CI, CF, CF, B, gamma, V, FI, FI, FF, FF, FI, FF,
                                     ws, rneed - 1, nullptr) == SV_ERR_WORKSPACE);
    const sv_status na = sv_verify_chain_noalloc(F, F, dt, CI, CF, CF, B, gamma, V, FI, FI,
                                                 nullptr, nullptr, nullptr, nullptr);
    CHECK_AT(na == (need <= SV_NOALLOC_SCRATCH_BYTES ? SV_OK : SV_ERR_SCRATCH),
             "noalloc B=%d gamma=%d V=%lld: status %d, workspace %zu", B, gamma, (long long)V,
             int(na), need);
    const size_t gneed = sv_verify_chain_greedy_workspace_bytes(B, gamma, V, dt);
    g_ws_bytes = gneed;
    CHECK(gneed > 0 && sv_verify_chain_greedy(F, dt, CI, B, gamma, V, FI, FI, FI, FI, kFake,
                                              gneed, nullptr) == SV_OK);
    const size_t aneed = sv_chain_acceptance_rates_workspace_bytes(B, gamma, V, dt);
    g_ws_bytes = aneed;
    const sv_status ast = sv_chain_acceptance_rates(F, F, dt, CF, B, gamma, V, FF, FI, kFake,
                                                    aneed, nullptr);
    CHECK_AT(aneed > 0 && ast == SV_OK, "rates B=%d gamma=%d V=%lld: status %d, workspace %zu",
             B, gamma, (long long)V, int(ast), aneed);
  }
}

void tree(int32_t n_trees, int32_t n_nodes, int64_t V, sv_status want) {
  const size_t need = sv_verify_tree_workspace_bytes(n_trees, n_nodes, V, SV_BF16);
  g_ws_bytes = need;
  const long before = g_launches;
  const sv_status st = sv_verify_tree(F, SV_BF16, CI, CI, n_trees, n_nodes, V, FI, FI, FI, FI,
                                      FI, kFake, need, nullptr);
  CHECK_AT(st == want, "tree %d x %d V=%lld: status %d, want %d", n_trees, n_nodes,
           (long long)V, int(st), int(want));
  CHECK((g_launches > before) == (st == SV_OK));
  CHECK((need > 0) == (want == SV_OK));
}

void sample(int32_t rows, int64_t V, sv_status want) {
  const size_t need = sv_sample_workspace_bytes(rows, V, SV_F32);
  g_ws_bytes = need;
  const sv_status st = sv_sample(F, SV_F32, CF, CF, rows, V, FI, FF, FI, kFake, need, nullptr);
  CHECK_AT(st == want, "sample rows=%d V=%lld: status %d, want %d", rows, (long long)V, int(st),
           int(want));
}

void kv(int64_t row_bytes, int32_t n, int32_t src_rows, int32_t dst_rows, sv_status want,
        const void* src = F, void* dst = reinterpret_cast<void*>(uintptr_t(1) << 60)) {
  const long before = g_launches;
  const sv_status st = sv_compact_accepted(src, dst, row_bytes, n, src_rows, dst_rows, CI, 8, CI,
                                           CI, FI, nullptr);
  CHECK_AT(st == want, "kv row_bytes=%lld n=%d rows %d/%d: status %d, want %d",
           (long long)row_bytes, n, src_rows, dst_rows, int(st), int(want));
  CHECK((g_launches > before) == (st == SV_OK));
}

}  // namespace

int main() {
  const int64_t VMAX = INT32_MAX;

  // ---- chain: every validation path
  chain(1, 4, 1000, SV_OK, SV_F32);
  CHECK(sv_verify_chain(nullptr, F, SV_F32, CI, CF, CF, 1, 4, 1000, FI, FI, FF, FF, FI, kFake,
                        1 << 20, nullptr) == SV_ERR_NULL);
  CHECK(sv_verify_chain(F, F, SV_F32, CI, CF, CF, 1, 4, 1000, nullptr, FI, FF, FF, FI, kFake,
                        1 << 20, nullptr) == SV_ERR_NULL);
  CHECK(sv_verify_chain(F, F, sv_dtype(7), CI, CF, CF, 1, 4, 1000, FI, FI, FF, FF, FI, kFake,
                        1 << 20, nullptr) == SV_ERR_DTYPE);
  for (int32_t B : {0, -1, sv::kMaxBatch + 1, 1 << 24}) chain(B, 4, 1000, SV_ERR_SHAPE);
  for (int32_t g : {0, -3, 65, INT32_MAX}) chain(2, g, 1000, SV_ERR_SHAPE);
  for (int64_t V : {int64_t(0), int64_t(-5), VMAX + 1, INT64_MAX}) chain(2, 4, V, SV_ERR_SHAPE);
  chain(3, 4, 5000, SV_ERR_WORKSPACE, SV_BF16, 256);                     // too small
  chain(3, 4, 5000, SV_ERR_WORKSPACE, SV_BF16, 0, nullptr);              // missing
  chain(3, 4, 5000, SV_ERR_WORKSPACE, SV_BF16, 0, kFake + 16);           // misaligned
  CHECK(sv_verify_chain_workspace_bytes(3, 4, 5000, sv_dtype(9)) == 0);

  // ---- chain: the shape limits and a sweep up to them
  chain(sv::kMaxBatch, 1, 1, SV_OK);
  chain(1, 64, VMAX, SV_ERR_SHAPE);               // 129 * 2^20 chunks: past 2^32 work-items
  chain(1, 64, int64_t(1) << 29, SV_OK);          // 129 * 2^18 chunks
  chain(sv::kMaxBatch, 64, 1, SV_ERR_SHAPE);      // 2^22 * 129 one-wave chunks
  chain(1 << 18, 64, 1, SV_OK);                   // 2^18 * 129 chunks < 2^26
  for (int32_t B : {1, 3, 255, 256, 4096, 65535, 1 << 20, sv::kMaxBatch})
    for (int32_t g : {1, 4, 7, 31, 64})
      for (int64_t V : {int64_t(1), int64_t(2047), int64_t(2049), int64_t(152064),
                        int64_t(1) << 24, VMAX}) {
        // Independent statement of the limit: every chunk a wave, rounded up to 16-wave groups,
        // and one 1024-thread workgroup per sequence, each launch below 2^32 work-items.
        const int64_t chunks = int64_t(B) * (2 * g + 1) * ((V + 2047) / 2048);
        const bool fits = (chunks + 15) / 16 * 1024 < (int64_t(1) << 32) &&
                          int64_t(B) * 1024 < (int64_t(1) << 32);
        chain(B, g, V, fits ? SV_OK : SV_ERR_SHAPE);
      }

  // ---- tree
  tree(16, 64, 32000, SV_OK);
  tree(1, 4096, VMAX, SV_ERR_SHAPE);  // 2^32 chunks
  tree(1, 4096, int64_t(1) << 24, SV_OK);         // 2^25 chunks
  tree(4, 4096, int64_t(1) << 24, SV_ERR_SHAPE);
  tree(1, 4097, 100, SV_ERR_SHAPE);
  tree(0, 64, 100, SV_ERR_SHAPE);
  tree(sv::kMaxBatch, 1, 1, SV_OK);
  tree(sv::kMaxBatch + 1, 1, 1, SV_ERR_SHAPE);
  tree(1 << 16, 1024, 1, SV_ERR_SHAPE);     // 2^26 one-wave chunks
  tree((1 << 16) - 1, 1024, 1, SV_OK);
  CHECK(sv_verify_tree(F, SV_BF16, nullptr, CI, 1, 8, 100, FI, FI, FI, FI, FI, kFake, 1 << 20,
                       nullptr) == SV_ERR_NULL);
  g_ws_bytes = 1 << 20;
  CHECK(sv_verify_tree(F, SV_BF16, CI, CI, 1, 8, 100, FI, FI, FI, FI, FI, kFake, 16, nullptr) ==
        SV_ERR_WORKSPACE);

  // ---- sampler
  sample(1, 1, SV_OK);
  sample(256, 152064, SV_OK);
  sample(sv::kMaxBatch, 1, SV_OK);
  sample(sv::kMaxBatch + 1, 1, SV_ERR_SHAPE);
  sample(INT32_MAX, 1, SV_ERR_SHAPE);
  sample(1, VMAX, SV_OK);
  sample(64, VMAX, SV_ERR_SHAPE);
  sample(0, 100, SV_ERR_SHAPE);

  // ---- KV compaction: sizes whose products leave int64 must be refused, not wrap
  kv(131072, 256, 8, 64, SV_OK);
  kv(int64_t(1) << 40, 1, 1, 1, SV_ERR_SHAPE);                   // 8 * 2^31 tiles
  kv(int64_t(1) << 29, 1, 1, 1, SV_OK);                          // 8 * 2^20 tiles of 512 B
  kv(int64_t(1) << 30, 1, 1, 1, SV_ERR_SHAPE);                   // 2^32 work-items
  kv((int64_t(1) << 40) + 1, 1, 1, 1, SV_ERR_SHAPE);
  kv(INT64_MAX, 1, 1, 1, SV_ERR_SHAPE);
  kv(int64_t(1) << 40, INT32_MAX, INT32_MAX, 1, SV_ERR_SHAPE);  // n * src_rows * row_bytes
  kv(int64_t(1) << 40, INT32_MAX, 1, INT32_MAX, SV_ERR_SHAPE);
  kv(int64_t(1) << 30, INT32_MAX, 1, 1, SV_ERR_SHAPE);          // n * 8 * tiles
  kv(1, (1 << 21) - 1, 1, 1, SV_OK);                              // n * 8 * 256 < 2^32
  kv(1, 1 << 21, 1, 1, SV_ERR_SHAPE);
  kv(16, 4, 8, 8, SV_ERR_SHAPE, F, kFake + 64);                  // overlapping buffers
  kv(0, 4, 8, 8, SV_ERR_SHAPE);
  kv(16, 0, 8, 8, SV_ERR_SHAPE);

  // ---- read probe
  CHECK(sv_read_probe_out_words(0) == 0 && sv_read_probe_out_words(15) == 0);
  CHECK(sv_read_probe_out_words(INT64_MAX - 15) == 0);  // past 2^32 work-items
  CHECK(sv_read_probe_out_words(int64_t(1) << 40) == 0);  // 2^23 groups of 1024 threads
  CHECK(sv_read_probe_out_words(int64_t(1) << 36) == size_t(1) << 19);
  CHECK(sv_read_probe_out_words(16) == 1);
  CHECK(sv_read_probe(F, 1 << 20, reinterpret_cast<uint32_t*>(kFake), nullptr) == SV_OK);
  CHECK(sv_read_probe(F, 17, reinterpret_cast<uint32_t*>(kFake), nullptr) == SV_ERR_SHAPE);

  // ---- status strings
  for (int s = 0; s <= 8; ++s) CHECK(sv_status_string(sv_status(s)) != nullptr);

  printf("abi_check: %ld checks, %ld launches, %d failed\n", g_checks, g_launches, g_fail);
  return g_fail == 0 ? 0 : 1;
}
