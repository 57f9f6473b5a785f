"""GPU results inside the parity bands, on purpose.

Rows are built so that an accept test or a draw falls inside the 1e-6 band where fp32-level
rounding may legitimately flip the integer outcome:

* accept band: the uniform of position i0 is the fp32 value within 5e-7 of the oracle's
  min(1, p/q) at that position (earlier positions get u = 0, so they accept), the strict test of
  the Speculative Sampling explainer's Step 3 (ステップ3);
* edge band: the draw's uniform puts u * W within 5e-7 * W of a bucket edge of the inverse CDF,
  for residual draws (modified rejection sampling, 修正付き棄却サンプリング) and bonus draws; half
  of the edges are the last positive-weight token of a chunk of 2048 elements, where the kernels'
  chunk search meets their in-chunk scan.

Every such row must be counted in its band by the oracle, and the GPU's outcome must be in the
allowed set (tests/parity.py): the oracle replayed with either decision, or a token whose
bucket lies within the band.  Run on the three eager chain paths, both early-exit forms and the
sampler.  The counts, and how many band rows came out other than the oracle's own outcome, are
printed.
"""

import numpy as np
import pytest
import torch

from oracle import chain as OC
from oracle import sample as OS
from parity import chain_refs, check_chain, check_sample
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu

DELTAS = [-5e-7, -1e-7, -3e-8, 0.0, 3e-8, 1e-7, 5e-7]
CHUNK = 2048


def _edge_uniform(w, rng, i, at_chunk_end):
    """An fp32 uniform u with u * W within 5e-7 * W of an upper bucket edge C(x) of weights w:
    x the last positive-weight token of a chunk (at_chunk_end) or a random one, with C(x) / W
    away from 0 and 1."""
    c = np.cumsum(w)
    total = c[-1]
    pos = np.flatnonzero(w > 0)
    ok = pos[(c[pos] / total > 0.02) & (c[pos] / total < 0.98)]
    if at_chunk_end:
        ends = [int(ok[ok // CHUNK == ch][-1]) for ch in np.unique(ok // CHUNK)
                if (ok // CHUNK == ch).any()]
        ends = [x for x in ends if x < len(w) - 1]
        if ends:
            ok = np.array(ends)
    x = int(ok[rng.integers(len(ok))])
    u = np.float32(c[x] / total + DELTAS[i % len(DELTAS)])
    return float(u)


def band_chain(seed, B, gamma, V, dtype):
    """A Gaussian chain batch whose uniforms are moved into the bands: sequences with s % 3 == 0
    put position s % gamma in the accept band, s % 3 == 1 put the residual draw on an edge, and
    s % 3 == 2 accept every draft and put the bonus draw on an edge.  Returns the batch and the
    band kind each sequence was built for."""
    b = I.chain_gaussian(seed, B, gamma, V, dtype, 2.0, 1.0, 1.0)
    rng = np.random.default_rng(seed + 1)
    kinds = []
    for s in range(B):
        zt = OC.widen(b.target[s], dtype)
        zd = OC.widen(b.draft[s], dtype)
        u = b.uniforms[s].astype(np.float64)
        toks, T = b.draft_tokens[s], float(b.temperature[s])
        if s % 3 == 0:
            res = OC.verify_chain_seq(zt, zd, toks, u, T)
            thr = np.minimum(1.0, res["p_at"] / res["q_at"])
            cands = [i for i in range(gamma) if thr[i] < 0.999] or [s % gamma]
            i0 = cands[s % len(cands)]
            u[:i0] = 0.0
            u[i0] = float(np.float32(thr[i0] + DELTAS[s % len(DELTAS)]))
            kinds.append(("accept_band", i0))
        elif s % 3 == 1:
            res = OC.verify_chain_seq(zt, zd, toks, u, T)
            if res["k"] == gamma:  # make it reject at position 0
                u[0] = 0.9999
                res = OC.verify_chain_seq(zt, zd, toks, u, T)
            u[gamma] = _edge_uniform(res["weights"], rng, s, at_chunk_end=(s // 3) % 2 == 0)
            kinds.append(("edge_band", res["k"]))
        else:
            u[:gamma] = 0.0
            res = OC.verify_chain_seq(zt, zd, toks, u, T)
            u[gamma] = _edge_uniform(res["weights"], rng, s, at_chunk_end=(s // 3) % 2 == 0)
            kinds.append(("edge_band", gamma))
        b.uniforms[s] = u.astype(np.float32)
    return b, kinds


def expected_counts(b, kinds, refs):
    """Each row's flag, from the oracle, must be the band it was built for."""
    want = {"accept_band": 0, "edge_band": 0}
    for s, (kind, pos) in enumerate(kinds):
        r = refs[s]
        if kind == "accept_band":
            assert pos in r["flag_accept"], (s, pos, r["flag_accept"])
        else:
            assert r["edge"] < OC.BAND and not r["flag_accept"], (s, r["edge"], r["flag_accept"])
            assert r["k"] == pos, (s, r["k"], pos)
        want[kind] += 1
    return want


def run_chain(b, lazy=False):
    d = BD.chain_to_device(b)
    out = BD.sv_verify_chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"],
                             d["temperature"], lazy=lazy)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


CASES = [(31, 42, 4, 5000, "f32"), (32, 42, 4, 5000, "bf16"), (33, 21, 7, 4100, "f32")]
_BUILT = {}


def built(case):
    if case not in _BUILT:
        b, kinds = band_chain(*case)
        refs = chain_refs(b)
        _BUILT[case] = (b, kinds, refs, expected_counts(b, kinds, refs))
    return _BUILT[case]


@pytest.mark.parametrize("path", ["fused", "finish", "split", "lazy", "staged"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[4]}_B{c[1]}_g{c[2]}_V{c[3]}")
def test_chain_rows_in_bands(case, path, monkeypatch):
    monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", path)
    b, kinds, refs, want = built(case)
    lazy = path in ("lazy", "staged")
    out = run_chain(b, lazy=lazy)
    counts = check_chain(b, out, lazy=lazy, refs=refs)
    print(f"[bands] {path} {case}: {counts}", flush=True)
    assert counts["accept_band"] == want["accept_band"]
    assert counts["edge_band"] == want["edge_band"]
    assert counts["exact"] == 0 and counts["fallback"] == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sampler_rows_in_edge_band(dtype):
    s = I.sample_gaussian(34, 48, 6000, dtype, 2.5, 0.8)
    rng = np.random.default_rng(35)
    for r in range(s.rows):
        res = OS.sample_row(OC.widen(s.logits[r], dtype), s.temperature[r], s.uniforms[r])
        s.uniforms[r] = _edge_uniform(res["weights"], rng, r, at_chunk_end=r % 2 == 0)
        again = OS.sample_row(OC.widen(s.logits[r], dtype), s.temperature[r], s.uniforms[r])
        assert again["edge"] < OC.BAND, (r, again["edge"])
    d = BD.sample_to_device(s)
    out = BD.sv_sample(d["logits"], d["temperature"], d["uniforms"])
    torch.cuda.synchronize()
    counts = check_sample(s, {k: v.cpu().numpy() for k, v in out.items()})
    print(f"[bands] sampler {dtype}: {counts}", flush=True)
    assert counts["edge_band"] == s.rows
