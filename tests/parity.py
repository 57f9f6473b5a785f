"""GPU-versus-oracle comparison rules (shared by the parity tests, the smoke check and the bench).

Integer outputs must be bit-exact, except where the oracle itself reports that fp32-level
rounding may flip the decision:

* an accept test with |u - min(1, p/q)| < 1e-6: the GPU result must equal the oracle
  replayed with either decision at each such position;
* a draw with u*W within 1e-6*W of a bucket edge: the GPU token must be one whose bucket
  lies within 1e-6*W of u*W (oracle.chain.draw_band): the oracle's token, or the nearest
  positive-weight token across an edge that lies within the band (beyond it only when that
  neighbour's whole bucket is narrower than the band).

Rows inside a band are counted by kind ("accept_band", "edge_band"); "band_differs" counts
those where the GPU returned an outcome other than the oracle's own.

Probabilities p_i(x_i), q_i(x_i) must satisfy |gpu - ref| <= 1e-5 * ref + 1e-30.
"""

from __future__ import annotations

import itertools

import numpy as np

from oracle import alpha as OA
from oracle import chain as OC
from oracle import greedy as OG
from oracle import kv as OK
from oracle import sample as OS
from oracle import tree as OT

P_RTOL = 1e-5
P_ATOL = 1e-30
# Acceptance rates: |gpu - ref| <= 1e-5 * ref + 1e-12 (fp32 terms, fp64 sums; min is
# 1-Lipschitz, so the terms' relative error carries over unamplified).
ALPHA_RTOL = 1e-5
ALPHA_ATOL = 1e-12


# Band rows allowed per full-size workload: twice the count its seeded inputs give (the accept
# band and the edge band together, as tests/record_parity.py records them), so that a change
# that widened the bands, or moved many rows into them, fails the parity tests.  At most a
# quarter of that many (and at least 2) band rows may be resolved differently from the oracle.
BAND_LIMITS = {
    "zipf_b64_g4_v128256_bf16": 8,      # recorded: 4 edge-band rows of 64
    "gauss_b256_g7_v152064_f32": 16,    # recorded: 8 edge-band rows of 256
    "sample_b256_v152064_f32": 48,      # recorded: 24 of 256 rows
    "sample_b64_v128256_bf16": 12,      # recorded: 6 of 64 rows
}


def assert_band_limit(name, counts):
    """The band counts of a full-size workload stay within BAND_LIMITS."""
    limit = BAND_LIMITS[name]
    bands = counts.get("accept_band", 0) + counts["edge_band"]
    assert bands <= limit, f"{name}: {bands} band rows, more than {limit}: {counts}"
    assert counts["band_differs"] <= max(2, limit // 4), f"{name}: {counts}"


def allowed_outcomes(target, draft, toks, uni, temp, res):
    """(k, tokens) pairs the GPU may return for this sequence, with a flag kind."""
    kind = "exact"
    cands = [res]
    if res["flag_accept"]:
        kind = "accept_band"
        cands = []
        flagged = res["flag_accept"]
        for bits in itertools.product([False, True], repeat=len(flagged)):
            force = dict(zip(flagged, bits))
            cands.append(OC.verify_chain_seq(target, draft, toks, uni, temp, force=force))
    allowed = set()
    u_draw = float(uni[-1])
    for r in cands:
        if r["edge"] < OC.BAND:
            if kind == "exact":
                kind = "edge_band"
            for y in OC.draw_band(r["weights"], u_draw):
                allowed.add((r["k"], tuple(r["tokens"][:-1]) + (y,)))
        else:
            allowed.add((r["k"], tuple(r["tokens"])))
    return allowed, kind


def chain_refs(batch, seqs=None):
    """The oracle's result for each listed sequence of a chain batch ({b: result}), for tests
    that compare several GPU runs of one batch with the oracle."""
    seqs = range(batch.B) if seqs is None else seqs
    return {b: OC.verify_chain_seq(OC.widen(batch.target[b], batch.dtype),
                                   OC.widen(batch.draft[b], batch.dtype), batch.draft_tokens[b],
                                   batch.uniforms[b], batch.temperature[b]) for b in seqs}


def check_chain(batch, out, seqs=None, lazy=False, refs=None):
    """Compare GPU chain outputs (numpy arrays) with the oracle on the listed sequences.

    out: dict with tokens [B, gamma+1], num_accepted [B], p, q [B, gamma], status [B].
    lazy: outputs of the early-exit entry point, whose p and q after the cut k are either NaN
    (row not read) or the evaluated values; positions i <= k are checked as usual.
    refs: the oracle's results from chain_refs (computed here when absent).
    Returns counts {"exact": n, "accept_band": n, "edge_band": n, "fallback": n,
    "band_differs": n} (the last: band rows whose GPU outcome is not the oracle's own).
    Raises AssertionError with a description on the first mismatch.
    """
    B, gamma = batch.B, batch.gamma
    seqs = range(B) if seqs is None else seqs
    counts = {"exact": 0, "accept_band": 0, "edge_band": 0, "fallback": 0, "band_differs": 0}
    for b in seqs:
        zt = OC.widen(batch.target[b], batch.dtype)
        zd = OC.widen(batch.draft[b], batch.dtype)
        toks, uni, temp = batch.draft_tokens[b], batch.uniforms[b], batch.temperature[b]
        res = refs[b] if refs is not None else OC.verify_chain_seq(zt, zd, toks, uni, temp)
        st = int(out["status"][b])
        assert st == res["status"], f"seq {b}: status {st} != oracle {res['status']}"
        k = int(out["num_accepted"][b])
        row = [int(x) for x in out["tokens"][b]]
        assert all(x == -1 for x in row[k + 1:]), f"seq {b}: padding {row}"
        if res["status"] & OC.FALLBACK_BITS:
            assert k == 0 and row[0] == 0, f"seq {b}: fallback expected, got k={k} {row}"
            counts["fallback"] += 1
            continue
        # probabilities
        for name, ref in (("p", res["p_at"]), ("q", res["q_at"])):
            got = np.asarray(out[name][b], dtype=np.float64)
            if lazy:
                tail = slice(k + 1, None)
                assert np.all(np.isnan(got[tail]) | (np.abs(got[tail] - ref[tail])
                                                     <= P_RTOL * np.abs(ref[tail]) + P_ATOL)), \
                    f"seq {b}: {name} after the cut {got[tail]} oracle {ref[tail]}"
                got, ref = got[:k + 1], ref[:k + 1]
            err = np.abs(got - ref)
            lim = P_RTOL * np.abs(ref) + P_ATOL
            bad = np.flatnonzero(~(err <= lim))
            assert len(bad) == 0, (f"seq {b}: {name}[{bad[0]}] gpu {got[bad[0]]!r} "
                                   f"oracle {ref[bad[0]]!r}")
        allowed, kind = allowed_outcomes(zt, zd, toks, uni, temp, res)
        got = (k, tuple(row[:k + 1]))
        assert got in allowed, (f"seq {b} ({kind}): gpu k={k} tokens={row[:k + 1]} "
                                f"oracle k={res['k']} tokens={res['tokens']} "
                                f"edge={res['edge']:.3g} flags={res['flag_accept']}")
        counts[kind] += 1
        if got != (res["k"], tuple(res["tokens"])):
            counts["band_differs"] += 1
    return counts


def check_tree(batch, out, trees=None):
    """Compare GPU tree outputs with the oracle: bit-exact path, tokens, k, argmax, status."""
    n = batch.n_nodes
    trees = range(batch.n_trees) if trees is None else trees
    accepted = []
    for t in trees:
        res = OT.verify_tree_one(OC.widen(batch.logits[t], batch.dtype), batch.parents[t],
                                 batch.node_tokens[t])
        k = res["k"]
        assert int(out["status"][t]) == res["status"], f"tree {t}: status"
        assert int(out["num_accepted"][t]) == k, f"tree {t}: k {out['num_accepted'][t]} != {k}"
        path = list(res["path"]) + [-1] * (n - len(res["path"]))
        toks = list(res["tokens"]) + [-1] * (n - len(res["tokens"]))
        assert [int(x) for x in out["path"][t]] == path, f"tree {t}: path"
        assert [int(x) for x in out["tokens"][t]] == toks, f"tree {t}: tokens"
        if out.get("node_argmax") is not None:
            assert [int(x) for x in out["node_argmax"][t]] == res["g"], f"tree {t}: argmax"
        accepted.append(k)
    return accepted


def check_chain_greedy(batch, out, seqs=None):
    """Compare GPU greedy chain outputs (numpy arrays) with the oracle, bit-exact.

    out: dict with tokens [B, gamma+1], num_accepted [B], argmax [B, gamma+1] (or None),
    status [B].  Returns the list of accepted counts.
    """
    B, gamma = batch.B, batch.gamma
    seqs = range(B) if seqs is None else seqs
    ks = []
    for b in seqs:
        res = OG.verify_chain_greedy_seq(OC.widen(batch.target[b], batch.dtype),
                                         batch.draft_tokens[b])
        want = res["tokens"] + [-1] * (gamma + 1 - len(res["tokens"]))
        got = [int(x) for x in out["tokens"][b]]
        assert int(out["num_accepted"][b]) == res["k"], (b, int(out["num_accepted"][b]), res)
        assert got == want, (b, got, want)
        assert int(out["status"][b]) == res["status"], (b, int(out["status"][b]), res["status"])
        if out.get("argmax") is not None:
            assert [int(x) for x in out["argmax"][b]] == res["g"], (b, out["argmax"][b], res["g"])
        ks.append(res["k"])
    return ks


def check_acceptance_rates(batch, out, seqs=None):
    """Compare GPU acceptance rates with the oracle: values within ALPHA_RTOL / ALPHA_ATOL (NaN
    where the oracle gives NaN), status bits exact.  Returns the list of alpha arrays."""
    seqs = range(batch.B) if seqs is None else seqs
    res = []
    for b in seqs:
        al, st = OA.acceptance_rates_seq(OC.widen(batch.target[b], batch.dtype),
                                         OC.widen(batch.draft[b], batch.dtype),
                                         batch.temperature[b])
        got = np.asarray(out["alpha"][b], dtype=np.float64)
        nan = np.isnan(al)
        assert np.array_equal(nan, np.isnan(got)), (b, got, al)
        err = np.abs(got[~nan] - al[~nan])
        assert np.all(err <= ALPHA_RTOL * al[~nan] + ALPHA_ATOL), (b, got, al, err)
        if out.get("status") is not None:
            assert [int(x) for x in out["status"][b]] == [int(x) for x in st], (b, out["status"][b], st)
        res.append(al)
    return res


def check_sample(batch, out, rows=None):
    """Compare GPU sampler outputs with the oracle: tokens bit-exact unless the oracle reports the
    draw within the 1e-6 band of a bucket edge (then a token whose bucket lies within the band,
    oracle.chain.draw_band), p(y) within the probability bound, status
    exact.  Returns {"exact": n, "edge_band": n, "fallback": n, "band_differs": n}."""
    rows = range(batch.rows) if rows is None else rows
    counts = {"exact": 0, "edge_band": 0, "fallback": 0, "band_differs": 0}
    for r in rows:
        res = OS.sample_row(OC.widen(batch.logits[r], batch.dtype), batch.temperature[r],
                            batch.uniforms[r])
        y = int(out["tokens"][r])
        assert int(out["status"][r]) == res["status"], (r, int(out["status"][r]), res["status"])
        if res["status"]:
            assert y == 0, (r, y)
            counts["fallback"] += 1
            continue
        if res["edge"] < OC.BAND:
            allowed = OC.draw_band(res["weights"], float(batch.uniforms[r]))
            assert y in allowed, (r, y, allowed)
            counts["edge_band"] += 1
            counts["band_differs"] += int(y != res["token"])
        else:
            assert y == res["token"], (r, y, res["token"])
            counts["exact"] += 1
        if out.get("prob") is not None:
            ref = float(res["weights"][y])
            assert abs(float(out["prob"][r]) - ref) <= P_RTOL * ref + P_ATOL, (r, out["prob"][r], ref)
    return counts


def check_kv(batch, dst_out, status):
    """GPU KV compaction against the oracle: the whole destination bytes exact, status exact."""
    ref = batch.dst_init.copy()
    st = OK.compact_batch(batch.src, ref, batch.paths, batch.num_accepted, batch.dst_start)
    assert np.array_equal(np.asarray(status), st), (status, st)
    for b in range(batch.n):
        assert np.array_equal(dst_out[b], ref[b]), f"sequence {b}: destination bytes differ"
    return st
