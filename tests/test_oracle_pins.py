"""Pins of the CPU oracle against facts that do not come from the oracle itself.

* Theorem 1 of the Speculative Sampling explainer (修正付き棄却サンプリング):
  every emitted token follows the target distribution.  Checked by chi-square
  against scipy's softmax on tiny vocabularies.
* The expected-speedup equation (期待される高速化): E[tokens per round] =
  (1 - alpha^(gamma+1)) / (1 - alpha) when every position has acceptance rate
  alpha = sum_x min(p(x), q(x)); the accept count A then has
  P(A=k) = alpha^k (1 - alpha) for k < gamma and P(A=gamma) = alpha^gamma.
* Special cases that reduce to library routines (p == q, disjoint supports,
  searchsorted for the inverse CDF, scipy's softmax, torch's bf16 widening).
* The worked examples under tests/golden/.
* Mutation checks: plausible mistakes planted in the oracle (on the CPU) make
  at least one pin fail.
"""

import json
import os

import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import softmax as sp_softmax

from oracle import chain as OC
from oracle import tree as OT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
P_MIN = 1e-3


# ----------------------------------------------------------------------------- helpers

def run_many(zt, zd, T, N, seed):
    """Oracle on N sequences sharing the logits, each with fresh draft tokens x_i ~ q_i
    (Gumbel-max on the draft logits) and fresh uniforms on the 2^-24 grid."""
    rng = np.random.default_rng(seed)
    g = zd.shape[0]
    ks = np.empty(N, dtype=np.int64)
    toks = []
    for n in range(N):
        x = np.argmax(zd / T + rng.gumbel(size=zd.shape), axis=1)
        u = rng.integers(0, 1 << 24, g + 1) / float(1 << 24)
        r = OC.verify_chain_seq(zt, zd, x, u, T)
        ks[n] = r["k"]
        toks.append(r["tokens"])
    return ks, toks


def theorem1_pvalues(zt, T, ks, toks, min_reached=400):
    """Chi-square p-value per emitted position j: the j-th emitted token, among sequences
    that emitted at least j+1 tokens, against p_j = softmax(z_t[j] / T) from scipy."""
    V = zt.shape[1]
    pv = []
    for j in range(zt.shape[0]):
        reached = [t[j] for t, k in zip(toks, ks) if k >= j]
        if len(reached) < min_reached:
            continue
        obs = np.bincount(reached, minlength=V)
        expct = sp_softmax(zt[j] / T) * len(reached)
        pv.append(stats.chisquare(obs, expct).pvalue)
    return pv


def closed_form(alpha, gamma):
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def accept_count_pvalue(ks, alpha, gamma):
    probs = np.array([alpha ** k * (1 - alpha) for k in range(gamma)] + [alpha ** gamma])
    obs = np.bincount(ks, minlength=gamma + 1)
    return stats.chisquare(obs, probs * len(ks)).pvalue


def mean_tokens_z(ks, alpha, gamma):
    emitted = ks + 1
    se = emitted.std(ddof=1) / np.sqrt(len(emitted))
    return abs(emitted.mean() - closed_form(alpha, gamma)) / se


def two_point_logits(a, b, gamma):
    """p = (a, 1-a) at every target row, q = (b, 1-b) at every draft row: alpha = 1 - |a - b|."""
    zt = np.log(np.array([[a, 1 - a]] * (gamma + 1)))
    zd = np.log(np.array([[b, 1 - b]] * gamma))
    return zt, zd


def random_logits(seed, gamma, V, noise=1.0):
    rng = np.random.default_rng(seed)
    zt = rng.normal(size=(gamma + 1, V))
    zd = zt[:gamma] + noise * rng.normal(size=(gamma, V))
    return zt, zd


# ----------------------------------------------------------------------------- primitives

def test_widen_bf16_matches_torch():
    rng = np.random.default_rng(0)
    f = rng.normal(scale=30.0, size=4096).astype(np.float32)
    f[:4] = [0.0, -0.0, np.inf, -np.inf]
    bits = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = OC.widen(bits, "bf16")
    assert np.array_equal(got, ref)
    assert np.array_equal(OC.widen(f, "f32"), f.astype(np.float64))


@pytest.mark.parametrize("T", [0.6, 1.0, 2.5])
def test_softmax_matches_scipy(T):
    rng = np.random.default_rng(1)
    z = rng.normal(scale=4.0, size=1000)
    z[::97] = -np.inf
    got = OC.softmax_fp64(z, T)
    ref = sp_softmax(z / T)
    assert np.allclose(got, ref, rtol=1e-12, atol=0)
    assert abs(got.sum() - 1.0) < 1e-12
    assert np.all(got[::97] == 0.0)


def test_inverse_cdf_matches_searchsorted():
    rng = np.random.default_rng(2)
    for _ in range(2000):
        V = int(rng.integers(1, 40))
        w = rng.random(V)
        w[rng.random(V) < 0.4] = 0.0
        if w.sum() == 0.0:
            w[int(rng.integers(0, V))] = 0.5
        u = rng.integers(0, 1 << 24) / float(1 << 24)
        y, edge = OC.inverse_cdf(w, u)
        c = np.cumsum(w)
        assert y == int(np.searchsorted(c, u * c[-1], side="right"))
        assert w[y] > 0.0
        assert 0.0 <= edge <= 1.0


def test_inverse_cdf_never_picks_zero_weight_at_u_zero():
    # u = 0 puts the target exactly on the left edge; the strict rule skips leading zeros.
    y, _ = OC.inverse_cdf(np.array([0.0, 0.0, 1.0, 1.0]), 0.0)
    assert y == 2


# ----------------------------------------------------------------------------- special cases

def test_hand_case_accept_and_reject():
    # p = (0.8, 0.2), q = (0.5, 0.5), drafted token 1: ratio 0.4.
    zt = np.log(np.array([[0.8, 0.2], [0.5, 0.5]]))
    zd = np.log(np.array([[0.5, 0.5]]))
    r = OC.verify_chain_seq(zt, zd, [1], [0.3, 0.75], 1.0)
    assert r["k"] == 1 and r["draw"] == "bonus" and r["tokens"] == [1, 1]
    assert abs(r["p_at"][0] - 0.2) < 1e-12 and abs(r["q_at"][0] - 0.5) < 1e-12
    for up in [0.0, 0.3, 0.999]:
        r = OC.verify_chain_seq(zt, zd, [1], [0.5, up], 1.0)
        # residual max(0, p - q) = (0.3, 0): only token 0 can come out.
        assert r["k"] == 0 and r["draw"] == "residual" and r["tokens"] == [0]


def test_p_equals_q_accepts_everything():
    rng = np.random.default_rng(3)
    gamma, V = 5, 50
    z = rng.normal(scale=2.0, size=(gamma + 1, V))
    for _ in range(200):
        x = rng.integers(0, V, gamma)
        u = rng.integers(0, 1 << 24, gamma + 1) / float(1 << 24)
        r = OC.verify_chain_seq(z, z[:gamma], x, u, 0.7)
        assert r["k"] == gamma and r["draw"] == "bonus"
        c = np.cumsum(sp_softmax(z[gamma] / 0.7))
        assert r["tokens"][-1] == int(np.searchsorted(c, u[gamma] * c[-1], side="right"))
        assert r["tokens"][:gamma] == list(x)


def test_disjoint_supports_reject_first_and_draw_from_p():
    # target mass on tokens {0, 1}, draft mass on {2, 3}: every draft is rejected at
    # position 0 and the residual equals p_0.
    ninf = -np.inf
    zt = np.array([[0.3, -0.4, ninf, ninf]] * 3)
    zd = np.array([[ninf, ninf, 0.0, 0.5]] * 2)
    ks, toks = run_many(zt, zd, 1.0, 4000, seed=4)
    assert np.all(ks == 0)
    ys = np.array([t[0] for t in toks])
    assert set(np.unique(ys)) <= {0, 1}
    p = sp_softmax(zt[0])
    assert stats.chisquare(np.bincount(ys, minlength=2)[:2], p[:2] * len(ys)).pvalue > P_MIN


# ----------------------------------------------------------------------------- Theorem 1

@pytest.mark.parametrize("V,gamma,T,seed", [(2, 3, 1.0, 10), (3, 4, 0.8, 11), (8, 3, 1.3, 12)])
def test_theorem1_emitted_tokens_follow_target(V, gamma, T, seed):
    zt, zd = random_logits(seed, gamma, V)
    ks, toks = run_many(zt, zd, T, 25000, seed=100 + seed)
    pv = theorem1_pvalues(zt, T, ks, toks)
    assert len(pv) >= 2
    assert min(pv) > P_MIN, pv


# ----------------------------------------------------------------------------- closed form

def test_closed_form_values():
    # E[tokens per round] at the acceptance rates the explainer's results table reports.
    assert abs(closed_form(0.70, 4) - 2.773100) < 1e-6
    assert abs(closed_form(0.72, 5) - 3.073878) < 1e-6
    assert abs(closed_form(0.85, 7) - 4.850063) < 1e-6
    assert abs(closed_form(0.65, 6) - 2.717079) < 1e-6


@pytest.mark.parametrize("a,b,gamma", [(0.6, 0.3, 4), (0.5, 0.35, 7)])
def test_closed_form_two_point(a, b, gamma):
    alpha = 1.0 - abs(a - b)
    zt, zd = two_point_logits(a, b, gamma)
    ks, _ = run_many(zt, zd, 1.0, 20000, seed=20 + gamma)
    assert mean_tokens_z(ks, alpha, gamma) < 4.0
    assert accept_count_pvalue(ks, alpha, gamma) > P_MIN


def test_closed_form_shifted_uniform_supports():
    # p uniform on {0..3}, q uniform on {1..4}: alpha = 3/4 at every position.
    gamma, ninf = 5, -np.inf
    zt = np.array([[0, 0, 0, 0, ninf]] * (gamma + 1), dtype=float)
    zd = np.array([[ninf, 0, 0, 0, 0]] * gamma, dtype=float)
    ks, toks = run_many(zt, zd, 1.0, 20000, seed=30)
    assert mean_tokens_z(ks, 0.75, gamma) < 4.0
    assert accept_count_pvalue(ks, 0.75, gamma) > P_MIN
    assert all(t[-1] != 4 for t in toks)  # token 4 has p = 0 and is never emitted


# ----------------------------------------------------------------------------- worked examples

def test_golden_sequence_diagram():
    g = json.load(open(os.path.join(GOLDEN, "p1_sequence_diagram.json")))
    s = g["scripted"]
    zt = np.log(np.array(s["target_probs"], dtype=np.float32)).astype(np.float64)
    zd = np.log(np.array(s["draft_probs"], dtype=np.float32)).astype(np.float64)
    r = OC.verify_chain_seq(zt, zd, s["draft_tokens"], s["uniforms"], s["temperature"])
    assert r["k"] == g["expected"]["num_accepted"] == 2
    assert r["tokens"] == g["expected"]["tokens"]
    assert len(r["tokens"]) == g["page_facts"]["tokens_fixed_in_round"]
    assert r["draw"] == g["expected"]["draw"]


def test_golden_greedy_example_as_tree():
    g = json.load(open(os.path.join(GOLDEN, "p2_greedy_example.json")))
    t = g["tree"]
    V = len(g["vocab"])
    logits = np.zeros((len(t["parents"]), V))
    for u, c in enumerate(t["target_choice_per_node"]):
        logits[u, c] = 5.0
    r = OT.verify_tree_one(logits, t["parents"], t["node_tokens"])
    assert r["path"] == g["expected"]["path"]
    assert r["k"] == g["expected"]["num_accepted"]
    assert r["tokens"] == g["expected"]["tokens"]
    assert [g["vocab"][x] for x in r["tokens"]] == g["page_facts"]["tokens_fixed_after_context"]


# ----------------------------------------------------------------------------- invariants and flags

def test_invariants_random():
    rng = np.random.default_rng(5)
    for trial in range(300):
        gamma = int(rng.integers(1, 8))
        V = int(rng.integers(1, 30))
        T = float(rng.choice([0.5, 1.0, 2.0]))
        zt, zd = random_logits(1000 + trial, gamma, V, noise=float(rng.random() * 3))
        x = np.argmax(zd / T + rng.gumbel(size=zd.shape), axis=1)
        u = rng.integers(0, 1 << 24, gamma + 1) / float(1 << 24)
        r = OC.verify_chain_seq(zt, zd, x, u, T)
        k = r["k"]
        assert 0 <= k <= gamma and len(r["tokens"]) == k + 1
        assert r["tokens"][:k] == list(x[:k])
        y = r["tokens"][-1]
        p = [sp_softmax(z / T) for z in zt]
        q = [sp_softmax(z / T) for z in zd]
        if r["draw"] == "bonus":
            assert k == gamma and p[gamma][y] > 0
        elif r["draw"] == "residual":
            assert max(0.0, p[k][y] - q[k][y]) > 0
        for i in range(k):
            assert u[i] < min(1.0, p[i][x[i]] / q[i][x[i]]) + 1e-12


def test_fallback_flags():
    zt, zd = random_logits(6, 3, 10)
    ok = dict(draft_tokens=[1, 2, 3], uniforms=[0.1, 0.2, 0.3, 0.4], temperature=1.0)

    def run(zt_=zt, zd_=zd, **kw):
        a = dict(ok)
        a.update(kw)
        return OC.verify_chain_seq(zt_, zd_, a["draft_tokens"], a["uniforms"], a["temperature"])

    assert run()["status"] == 0
    assert run(draft_tokens=[1, 10, 3])["status"] == OC.ROW_TOKEN_RANGE
    assert run(draft_tokens=[-1, 2, 3])["status"] == OC.ROW_TOKEN_RANGE
    assert run(temperature=0.0)["status"] == OC.ROW_BAD_TEMPERATURE
    assert run(temperature=float("nan"))["status"] == OC.ROW_BAD_TEMPERATURE
    assert run(uniforms=[0.1, 1.0, 0.3, 0.4])["status"] == OC.ROW_BAD_UNIFORM
    bad = zt.copy()
    bad[2, 4] = np.nan
    assert run(zt_=bad)["status"] == OC.ROW_NONFINITE
    bad = zd.copy()
    bad[1, :] = -np.inf
    r = run(zd_=bad)
    assert r["status"] == OC.ROW_NONFINITE and r["k"] == 0 and r["tokens"] == [0]


def test_residual_zero_fallback_draws_from_p():
    # x drafted with q(x) = 0 = p(x) forces a rejection at 0 while p_0 == q_0 elsewhere, so
    # max(0, p - q) is identically zero and the draw falls back to p_0.
    ninf = -np.inf
    zt = np.array([[0.0, 1.0, ninf], [0.0, 0.0, 0.0]])
    zd = np.array([[0.0, 1.0, ninf]])
    r = OC.verify_chain_seq(zt, zd, [2], [0.5, 0.9], 1.0)
    assert r["k"] == 0 and r["status"] == OC.ROW_RESIDUAL_ZERO
    c = np.cumsum(sp_softmax(zt[0]))
    assert r["tokens"] == [int(np.searchsorted(c, 0.9 * c[-1], side="right"))]


def test_accept_band_flag_and_force_replay():
    zt = np.log(np.array([[0.3, 0.7], [0.5, 0.5]]))
    zd = np.log(np.array([[0.6, 0.4]]))
    # ratio at token 0 is 0.5: u = 0.5 - 2^-24 lies inside the band
    u0 = 0.5 - 2.0 ** -24
    r = OC.verify_chain_seq(zt, zd, [0], [u0, 0.5], 1.0)
    assert r["flag_accept"] == [0]
    r2 = OC.verify_chain_seq(zt, zd, [0], [u0, 0.5], 1.0, force={0: not (r["k"] == 1)})
    assert r2["k"] != r["k"]


# ----------------------------------------------------------------------------- tree pins

def brute_force_tree(logits, parents, tokens):
    """Deepest root path whose every edge carries the parent's argmax (np.argmax), by
    enumerating every root-to-node path."""
    n = len(parents)
    g = [int(np.argmax(logits[u])) for u in range(n)]
    best = [0]
    for end in range(n):
        path = [end]
        while path[-1] != 0:
            path.append(parents[path[-1]])
        path = path[::-1]
        if all(tokens[path[i + 1]] == g[path[i]] for i in range(len(path) - 1)):
            if len(path) > len(best):
                best = path
    return best, [tokens[c] for c in best[1:]] + [g[best[-1]]]


def small_tree(rng, n, V, shape):
    if shape == "chain":
        parents = [-1] + list(range(n - 1))
    elif shape == "star":
        parents = [-1] + [0] * (n - 1)
    elif shape == "binary":
        parents = [-1] + [(i - 1) // 2 for i in range(1, n)]
    else:
        parents, kids = [-1], [0] * n
        for i in range(1, n):
            j = int(rng.choice([a for a in range(i) if kids[a] < V]))
            parents.append(j)
            kids[j] += 1
    tokens = [int(rng.integers(0, V))]
    for i in range(1, n):
        used = {tokens[c] for c in range(1, i) if parents[c] == parents[i]}
        free = [t for t in range(V) if t not in used]
        tokens.append(int(rng.choice(free)))
    return parents, tokens


@pytest.mark.parametrize("shape", ["chain", "star", "binary", "random"])
def test_tree_walk_matches_brute_force(shape):
    rng = np.random.default_rng(hash(shape) % 1000)
    for _ in range(300):
        n = int(rng.integers(1, 13))
        V = int(rng.integers(4, 9))
        if shape == "star":
            n = min(n, V)  # siblings carry distinct tokens
        parents, tokens = small_tree(rng, n, V, shape)
        logits = rng.integers(-2, 3, size=(n, V)).astype(np.float64)  # many ties
        r = OT.verify_tree_one(logits, parents, tokens)
        path, toks = brute_force_tree(logits, parents, tokens)
        assert r["path"] == path and r["tokens"] == toks and r["k"] == len(path) - 1


def test_argmax_first_matches_numpy_and_signed_zero():
    rng = np.random.default_rng(7)
    for _ in range(500):
        z = rng.integers(-3, 3, size=int(rng.integers(1, 50))).astype(np.float64)
        assert OT.argmax_first(z) == (int(np.argmax(z)), False)
    assert OT.argmax_first(np.array([-1.0, -0.0, 0.0]))[0] == 1
    assert OT.argmax_first(np.array([np.nan, 1.0, 2.0, 2.0])) == (2, True)


def test_tree_fallbacks():
    logits = np.zeros((3, 4))
    logits[0, 2] = 1.0
    r = OT.verify_tree_one(logits, [-1, 0, 5], [0, 2, 1])
    assert r["status"] == OC.ROW_BAD_TREE and r["path"] == [0] and r["tokens"] == [2]
    r = OT.verify_tree_one(logits, [-1, 0, 0], [0, 2, 4])
    assert r["status"] == OC.ROW_TOKEN_RANGE and r["tokens"] == [2]


# ----------------------------------------------------------------------------- mutation checks

def _theorem1_passes(V=3, gamma=3, T=0.8, seed=40, N=8000):
    zt, zd = random_logits(seed, gamma, V)
    ks, toks = run_many(zt, zd, T, N, seed=seed + 1)
    pv = theorem1_pvalues(zt, T, ks, toks, min_reached=200)
    return min(pv) > P_MIN


def _closed_form_passes(gamma=4, N=8000):
    zt, zd = two_point_logits(0.6, 0.3, gamma)
    ks, _ = run_many(zt, zd, 1.0, N, seed=41)
    return mean_tokens_z(ks, 0.7, gamma) < 4.0 and accept_count_pvalue(ks, 0.7, gamma) > P_MIN


def test_pins_pass_on_unmutated_oracle():
    assert _theorem1_passes() and _closed_form_passes()


MUTATIONS = {
    "residual_unclamped": ("residual_weights", lambda p, q: np.abs(p - q)),
    "residual_swapped": ("residual_weights", lambda p, q: np.maximum(0.0, q - p)),
    "ratio_transposed": ("accept_threshold",
                         lambda px, qx: (min(1.0, qx / px) if px > 0 else 1.0)),
    "accept_prob_halved": ("accept_threshold", lambda px, qx: 0.5 * min(1.0, px / qx)),
    "softmax_no_temperature": ("softmax_fp64", lambda z, T: sp_softmax(z)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_fail_a_pin(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(OC, attr, bad)
    try:
        ok = _theorem1_passes() and _closed_form_passes()
    except Exception:
        ok = False
    assert not ok, f"mutation {name} went undetected"


def _zero_weight_pin_passes():
    """u' = 0 with a zero-probability token first: the drawn token must have p > 0."""
    zt = np.array([[-np.inf, 0.0, 0.0], [-np.inf, 0.0, 0.0]])
    zd = np.array([[-np.inf, 0.0, 0.0]])
    r = OC.verify_chain_seq(zt, zd, [1], [0.0, 0.0], 1.0)
    return sp_softmax(zt[1])[r["tokens"][-1]] > 0.0


def test_zero_weight_pin():
    assert _zero_weight_pin_passes()


def test_planted_inverse_cdf_non_strict_fails(monkeypatch):
    def non_strict(w, u):
        c = np.cumsum(w)
        return int(np.argmax(c >= u * c[-1])), 1.0
    monkeypatch.setattr(OC, "inverse_cdf", non_strict)
    assert not _zero_weight_pin_passes()
