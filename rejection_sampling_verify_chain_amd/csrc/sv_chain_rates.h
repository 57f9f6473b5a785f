// Per-position acceptance rates (sv_chain_acceptance_rates, and after verification in
// sv_verify_chain_with_rates).  Source: the Speculative Sampling explainer (0h-n0.github.io,
// arXiv:2302.01318), Step 3 (ステップ3), the expected-speedup section (期待される高速化) and the
// monitoring list (監視・アラート).
//
// Included by sv_chain.hip only: the chain, acceptance-rate and sampler kernels form one
// translation unit, so every kernel template is instantiated and registered once.
#pragma once

namespace sv {
namespace {

// ------------------------------------------------------------------------------------ alpha

// Acceptance rate alpha_i = sum_x min(p_i(x), q_i(x)) of position i of sequence b (the Step 3
// accept probability averaged over x ~ q_i).  They follow a sweep whose partials hold, per
// sequence, tgt_rows target rows then gamma draft rows: target row i is partial row
// b * (tgt_rows + gamma) + i and draft row i is that plus tgt_rows (tgt_rows = gamma for the
// standalone acceptance rates, gamma + 1 when they follow chain verification, whose decide
// kernel has already merged the rows).  Kernels:
//   merge    one wave per row merges its chunk partials into (M, S) (standalone only).
//   overlap  one wave per (b, i, chunk c) adds s * sum_x min(ra e_t(x), rb e_d(x)) over chunk c
//            of target row i and draft row i, where e_t, e_d are the chunk-local softmax terms,
//            A and B the chunk scales taking them to p and q, s = max(A, B) and
//            (ra, rb) = (A, B) / s (one of them is 1, the other at most 1, so nothing
//            overflows); for bf16 rows with one exponential per element: min(ra e_t, rb e_d)
//            is 2 to the smaller of the two exponents, one of them offset by log2 of its
//            ratio.  A chunk where A or B is 0 adds nothing.  The chunk loads go out first;
//            the row statistics and chunk partials arrive through the scalar cache meanwhile.
//            Workgroups are sized like the sweep's (measured: 1024 threads for fp32, 256 for
//            bf16; a workgroup per (b, i) with waves looping over the chunks ran at 0.47 of
//            the HBM peak on 131 MB of bf16, this form at 0.68).
//   reduce   one wave per (b, i) adds the chunk sums in a fixed order (deterministic).
constexpr int kAlphaBlock = 256;
static_assert(kAlphaBlock <= kMaxBlock, "launch limits of the C ABI");

__device__ __forceinline__ int64_t alpha_target_row(const ChainParams& p, int64_t b, int i) {
  return b * (p.tgt_rows + p.gamma) + i;
}

__global__ __launch_bounds__(kAlphaBlock) void k_chain_alpha_merge(ChainParams p, int64_t rows) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = int64_t(blockIdx.x) * (kAlphaBlock / kWave) + wave_id();
  if (r >= rows) return;  // wave-uniform
  const int64_t b = r / (p.tgt_rows + p.gamma);
  const double Td = effective_temperature(uniform_load(p.temp, b));
  const RowStat st = merge_row(p.part + r * p.nchunk, p.nchunk, lane, Td);
  if (lane == 0) p.rowstat[r] = st;
}

// Waves per SIMD of the overlap kernel: five for 16-byte bf16 loads (at most 96 VGPRs); the
// fp32 kernel's 1024-thread workgroup already implies four, and the one-element-load form is
// left unbounded.
template <typename T, int VW>
constexpr int kAlphaWavesPerSimd = sizeof(T) == 2 && VW > 1 ? 5 : 1;

template <typename T, int VW>
__global__ __launch_bounds__(kStreamBlock<T>, (kAlphaWavesPerSimd<T, VW>)) void k_chain_alpha(ChainParams p, double* chunk_sum,
                                                                int64_t total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t w = int64_t(blockIdx.x) * (kStreamBlock<T> / kWave) + wave_id();
  if (w >= total) return;  // wave-uniform
  const int gamma = p.gamma;
  const int64_t V = p.V, nchunk = p.nchunk;
  const int64_t pair = w / nchunk;
  const int64_t c = w - pair * nchunk;
  const int64_t b = pair / gamma;
  const int i = int(pair - b * gamma);
  const int64_t jt = alpha_target_row(p, b, i), jd = jt + p.tgt_rows;  // rows of the partials
  const int nvalid = chunk_valid(V, c);
  RawChunk<T, VW> rt, rd;
  load_raw<T, VW>(static_cast<const T*>(p.tgt) + (b * (gamma + 1) + i) * V + c * kChunk, nvalid,
                  lane, rt);
  load_raw<T, VW>(static_cast<const T*>(p.drf) + (b * gamma + i) * V + c * kChunk, nvalid, lane,
                  rd);
  const float te = effective_temperature(uniform_load(p.temp, b));
  const double Td = te;
  const float kk = log2e_over_t(te);
  const RowStat st_t = uniform_load(p.rowstat, jt), st_d = uniform_load(p.rowstat, jd);
  const RowPart ct = uniform_load(p.part, jt * nchunk + c);
  const RowPart cd = uniform_load(p.part, jd * nchunk + c);
  double acc = 0.0;
  if (st_t.valid && st_d.valid) {  // wave-uniform
    const double A = chunk_scale(ct.m, st_t, Td), Bq = chunk_scale(cd.m, st_d, Td);
    if (A > 0.0 && Bq > 0.0) {  // wave-uniform; otherwise min(p, q) is 0 on the chunk
      float zt[kElemsPerLane], zd[kElemsPerLane];
      unpack_chunk<T, VW>(rt, nvalid, lane, zt);
      unpack_chunk<T, VW>(rd, nvalid, lane, zd);
      const double sc = fmax(A, Bq);
      if constexpr (sizeof(T) == 2) {
        // bf16 rows are short and bound by the per-element work: min(ra e_t, rb e_d) is taken
        // as 2^min(x_t + log2 ra, x_d + log2 rb), x = (z - m_c) log2(e) / T, one exponential
        // per element instead of two.  One of ra, rb is exactly 1 (log 0), so only the other
        // side takes an offset.  A ratio below 2^-149 gives -inf (a term of 0, as ra = 0 does
        // in the product form).
        double s;
        if (A < Bq) {  // wave-uniform
          const float off = log2f(float(A / sc));
          s = wave_sum(lane_term_sum([&](int e) {
            return hw_exp2(fminf((zt[e] - ct.m) * kk + off, (zd[e] - cd.m) * kk));
          }));
        } else {
          const float off = log2f(float(Bq / sc));
          s = wave_sum(lane_term_sum([&](int e) {
            return hw_exp2(fminf((zt[e] - ct.m) * kk, (zd[e] - cd.m) * kk + off));
          }));
        }
        acc = sc * s;
      } else {
        // fp32 rows are bound by HBM; the product form keeps the kernel's registers lower.
        const float ra = float(A / sc), rb = float(Bq / sc);
        acc = sc * wave_sum(lane_term_sum([&](int e) {
                return fminf(ra * softmax_term(zt[e], ct.m, kk), rb * softmax_term(zd[e], cd.m, kk));
              }));
      }
    }
  }
  if (lane == 0) chunk_sum[w] = acc;
}

__global__ __launch_bounds__(kAlphaBlock) void k_chain_alpha_reduce(ChainParams p,
                                                                   const double* chunk_sum,
                                                                   int64_t pairs, float* out_alpha,
                                                                   int32_t* out_status) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t pair = int64_t(blockIdx.x) * (kAlphaBlock / kWave) + wave_id();
  if (pair >= pairs) return;  // wave-uniform
  const int gamma = p.gamma;
  const int64_t nchunk = p.nchunk;
  const int64_t b = pair / gamma;
  const int64_t jt = alpha_target_row(p, b, int(pair - b * gamma)), jd = jt + p.tgt_rows;
  const double* cs = chunk_sum + pair * nchunk;
  double acc = 0.0;
  for (int64_t c0 = 0; c0 < nchunk; c0 += int64_t(kWave) * kMergeBatch) {
    double v[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int64_t c = c0 + int64_t(k) * kWave + lane;
      v[k] = c < nchunk ? cs[c] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) acc += v[k];
  }
  acc = wave_sum(acc);
  if (lane == 0) {
    const bool valid = uniform_load(p.rowstat, jt).valid && uniform_load(p.rowstat, jd).valid;
    out_alpha[pair] = valid ? float(acc) : NAN;
    if (out_status) {
      const float tb = uniform_load(p.temp, b);
      int bits = valid ? 0 : SV_ROW_NONFINITE;
      if (!(tb > 0.0f && tb < INFINITY)) bits |= SV_ROW_BAD_TEMPERATURE;
      out_status[pair] = bits;
    }
  }
}

// Overlap and reduce launches shared by the standalone acceptance rates and chain verification
// with rates (partials and row statistics already in the workspace).
template <typename T, int VW>
hipError_t launch_alpha_tail(const ChainParams& p, int64_t B, double* chunk_sum,
                             float* out_alpha, int32_t* out_status, hipStream_t s) {
  const int64_t pairs = B * p.gamma;
  const int64_t owaves = pairs * p.nchunk;
  constexpr int wpb = kStreamBlock<T> / kWave;
  hipError_t e = launch_kernel("alpha_overlap", k_chain_alpha<T, VW>,
                               dim3(unsigned(wave_groups(owaves, wpb))), dim3(kStreamBlock<T>), s,
                               p, chunk_sum, owaves);
  if (e != hipSuccess) return e;
  constexpr int awpb = kAlphaBlock / kWave;
  return launch_kernel("alpha_reduce", k_chain_alpha_reduce,
                       dim3(unsigned(wave_groups(pairs, awpb))), dim3(kAlphaBlock), s, p,
                       chunk_sum, pairs, out_alpha, out_status);
}

template <typename T, int VW>
hipError_t run_alpha(const AlphaArgs& a, hipStream_t s) {
  const AlphaLayout L = alpha_layout(a.B, a.gamma, a.V);
  ChainParams p = {};
  p.tgt = a.target;
  p.drf = a.draft;
  p.temp = a.temperature;
  p.gamma = a.gamma;
  p.tgt_rows = a.gamma;
  p.V = a.V;
  p.nchunk = L.nchunk;
  p.part = reinterpret_cast<RowPart*>(a.ws + L.off_part);
  p.rowstat = reinterpret_cast<RowStat*>(a.ws + L.off_rowstat);
  const int64_t rows = int64_t(a.B) * (2 * a.gamma);
  const int64_t total = rows * L.nchunk;
  const int64_t waves = (total + kUnitsPerWave<T> - 1) / kUnitsPerWave<T>;
  constexpr int wpb = kStreamBlock<T> / kWave;
  hipError_t e = launch_kernel("alpha_sweep", k_chain_sweep<T, VW>,
                               dim3(unsigned(wave_groups(waves, wpb))), dim3(kStreamBlock<T>), s,
                               p, total);
  if (e != hipSuccess) return e;
  constexpr int awpb = kAlphaBlock / kWave;
  e = launch_kernel("alpha_merge", k_chain_alpha_merge, dim3(unsigned(wave_groups(rows, awpb))),
                    dim3(kAlphaBlock), s, p, rows);
  if (e != hipSuccess) return e;
  return launch_alpha_tail<T, VW>(p, a.B, reinterpret_cast<double*>(a.ws + L.off_chunk_sum),
                                  a.out_alpha, a.out_status, s);
}

}  // namespace
}  // namespace sv
