// Draft-side sampler (sv_sample).  Source: the Speculative Sampling explainer (0h-n0.github.io,
// arXiv:2302.01318), Step 1 (ステップ1) and the code sketch's draft loop.
//
// Included by sv_chain.hip only: the chain, acceptance-rate and sampler kernels form one
// translation unit, so every kernel template is instantiated and registered once.
#pragma once

namespace sv {
namespace {

// ------------------------------------------------------------------------------------ sampler

// Draft-side sampler, one wave per logit row r: merges the row's chunk partials into (M, S),
// locates the chunk holding u * W from the chunk masses and rescans it in token order (the
// inverse CDF of the bonus draw), and evaluates p(y) in fp64.  Rows with a bad temperature,
// a bad uniform or no softmax take token 0.  For rows of up to 64 * kLocateBatch chunks the
// partials are loaded once and both the merge and the chunk masses come from those registers,
// and z(y) is taken from the rescanned chunk: two dependent memory round trips in all.
template <typename T, int VW>
__global__ __launch_bounds__(kWave) void k_sample_draw(ChainParams p, const float* uni,
                                                      int32_t* out_tokens, float* out_prob,
                                                      int32_t* out_status) {
  constexpr int NB = kLocateBatch;
  const int64_t r = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t V = p.V, nchunk = p.nchunk;
  const T* row = static_cast<const T*>(p.tgt) + r * V;
  const float tb = uniform_load(p.temp, r);
  const float te = effective_temperature(tb);
  const double Td = te;
  const float kk = log2e_over_t(te);
  const float uf = uniform_load(uni, r);
  const RowPart* pp = p.part + r * nchunk;
  const bool held = nchunk <= int64_t(kWave) * NB;  // uniform

  RowStat st;
  double w[NB];  // held rows: mass of chunk lane * NB + i
  if (held) {
    RowPart q[NB];
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t c = int64_t(lane) * NB + i;
      q[i] = c < nchunk ? pp[c] : RowPart{-INFINITY, 0, 0.0};
      mloc = fmaxf(mloc, q[i].m);
    }
    const float m = wave_max(mloc);
    const bool finite_max = (m > -INFINITY) && (m < INFINITY);
    double f[NB], s = 0.0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      f[i] = q[i].m == -INFINITY ? 0.0 : exp((double(q[i].m) - double(m)) / Td);
      s += q[i].s * f[i];  // a NaN partial survives the zero factor
    }
    s = finite_max ? wave_sum(s) : 0.0;
    st = RowStat{m, finite_max && (s > 0.0) && (s < INFINITY), s};
#pragma unroll
    for (int i = 0; i < NB; ++i) w[i] = q[i].s * (f[i] / s);  // q.s * chunk_scale
  } else {
    st = merge_row(pp, nchunk, lane, Td);
  }
  int status = 0;
  if (!(tb > 0.0f && tb < INFINITY)) status |= SV_ROW_BAD_TEMPERATURE;
  if (!(uf >= 0.0f && uf < 1.0f)) status |= SV_ROW_BAD_UNIFORM;
  if (!st.valid) status |= SV_ROW_NONFINITE;
  int64_t y = 0;
  double prob = NAN;
  if (status == 0) {
    const double u = uf;
    const Located at = held ? locate_chunk_held(w, lane, u)
                            : locate_chunk(nchunk, lane, u, [&](int64_t c) {
                                const RowPart q = pp[c];
                                return q.s * chunk_scale(q.m, st, Td);
                              });
    const int nvalid = chunk_valid(V, at.chunk);
    RawChunk<T, VW> raw;
    load_raw<T, VW>(row + at.chunk * kChunk, nvalid, lane, raw);
    const RowPart pc = uniform_load(pp, at.chunk);
    const double scale = chunk_scale(pc.m, st, Td);
    float z[kElemsPerLane];
    unpack_chunk<T, VW>(raw, nvalid, lane, z);
    const double tau_loc = scale > 0.0 ? (u * at.total - at.before) / scale : 0.0;
    y = chunk_scan<VW>(at.chunk, V, lane, tau_loc,
                       [&](int i) { return double(softmax_term(z[i], pc.m, kk)); });
    // z(y) from the lane that holds it: chunk offset o = (j * 64 + l) * VW + t.
    const int o = int(y - at.chunk * kChunk);
    const int slot = (o / (VW * kWave)) * VW + o % VW;
    float zy = z[0];
#pragma unroll
    for (int i = 1; i < kElemsPerLane; ++i) zy = i == slot ? z[i] : zy;
    zy = __shfl(zy, (o / VW) % kWave, kWave);
    prob = exp((double(zy) - double(st.m)) / Td) / st.s;
  }
  if (lane == 0) {
    out_tokens[r] = int32_t(y);
    if (out_prob) out_prob[r] = float(prob);
    if (out_status) out_status[r] = status;
  }
}

template <typename T, int VW>
hipError_t run_sample(const SampleArgs& a, hipStream_t s) {
  const SampleLayout L = sample_layout(a.rows, a.V);
  ChainParams p = {};
  p.tgt = a.logits;
  p.drf = a.logits;
  p.temp = a.temperature;
  p.gamma = 0;
  p.tgt_rows = 1;
  p.V = a.V;
  p.nchunk = L.nchunk;
  p.part = reinterpret_cast<RowPart*>(a.ws + L.off_part);
  const int64_t total = int64_t(a.rows) * L.nchunk;
  const int64_t waves = (total + kUnitsPerWave<T> - 1) / kUnitsPerWave<T>;
  constexpr int wpb = kStreamBlock<T> / kWave;
  hipError_t e = launch_kernel("sample_sweep", k_chain_sweep<T, VW>,
                               dim3(unsigned(wave_groups(waves, wpb))), dim3(kStreamBlock<T>), s,
                               p, total);
  if (e != hipSuccess) return e;
  return launch_kernel("sample_draw", k_sample_draw<T, VW>, dim3(unsigned(a.rows)), dim3(kWave),
                       s, p, a.uniforms, a.out_tokens, a.out_prob, a.out_status);
}

// Path choice for chain verification (all three give the same bits):
//   fused   one launch, one workgroup per sequence for every step;
//   finish  the sweep across the chip, then one workgroup per sequence for decide, residual and
//           draw (chain_finish);
//   split   the sweep, then decide, residual and draw as three launches.
// A 1024-thread workgroup (one per CU at its register count) streams about 128 KiB per memory
// round trip.  So the fused path wins when a sequence's rows take at most two such rounds, or
// when 192..256 sequences give every CU a workgroup and together they saturate HBM (the tails of
// some sequences then overlap the sweeps of others).  The finish path wins while a sequence's
// residual re-read (2 * V elements) stays small.  Measured per call, split / finish / fused:
// B = 1, V = 1000 fp32: 20.2 / 15.6 / 13.4 us; B = 64, V = 32000 bf16: 27.2 / 24.7 / 33.8 us;
// B = 256, V = 32000 bf16: 49.5 / 42.1 / 38.9 us; B = 256, gamma = 7, V = 152064 fp32:
// 406.8 / 400.8 / 390.4 us; B = 64, V = 128256 bf16: 48.1 / 54.4 / 103.1 us; B = 1, V = 152064
// fp32: 19.7 / 36.6 / 195.8 us; B = 1024, V = 32000 bf16: 141.4 / 144.0 / 145.0 us.
// Both one-workgroup forms need the sequence's partials and residual masses to fit their LDS
// budget; the rates need the sweep's partials in the workspace, so they take finish where fused
// would be chosen.  SPECVERIFY_CHAIN_PATH=fused, =finish or =split forces a path (for tests and
// measurement; subject to the LDS fit, and fused becomes finish with the rates).

}  // namespace
}  // namespace sv
