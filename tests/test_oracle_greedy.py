"""Pins of the greedy chain oracle against facts that do not come from it.

* The worked example of the ai-compass page (tests/golden/p2_greedy_example.json), read as a
  chain of four candidates.
* The zero-temperature limit of the stochastic verify: with a unique, well-separated maximum in
  every row and a temperature of 1e-3, p and q are one-hot in fp64, so the stochastic oracle
  (pinned by Theorem 1 and the closed form) must return the greedy result for any uniforms.
* The greedy walk over a chain-shaped token tree (the tree oracle is pinned by brute-force path
  enumeration), on integer logits with many ties.
* Mutation checks: plausible mistakes planted in the oracle make a pin fail.
"""

import json
import os

import numpy as np
import pytest

from oracle import chain as OC
from oracle import greedy as OG
from oracle import tree as OT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_greedy_example_as_chain():
    g = json.load(open(os.path.join(GOLDEN, "p2_greedy_example.json")))
    t = g["tree"]
    V = len(g["vocab"])
    choice = t["target_choice_per_node"]            # target's token after each node
    draft = t["node_tokens"][1:]                    # the four candidates
    logits = np.zeros((len(choice), V))
    for i, c in enumerate(choice):
        logits[i, c] = 5.0
    r = OG.verify_chain_greedy_seq(logits, draft)
    assert r["k"] == g["expected"]["num_accepted"] == 2
    assert r["tokens"] == g["expected"]["tokens"]
    assert [g["vocab"][x] for x in r["tokens"]] == g["page_facts"]["tokens_fixed_after_context"]
    discarded = [g["vocab"][x] for x in draft[r["k"]:] if g["vocab"][x] in g["page_facts"]["discarded"]]
    assert discarded == g["page_facts"]["discarded"]


def separated_logits(rng, rows, V):
    """Logits whose maximum is unique and at least 1 above the rest in every row."""
    z = rng.normal(0.0, 1.0, size=(rows, V))
    top = rng.integers(0, V, size=rows)
    for i in range(rows):
        z[i, top[i]] = z[i].max() + 1.0 + rng.random()
    return z


def _zero_temperature_agrees(seed=3, trials=400):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        gamma = int(rng.integers(1, 7))
        V = int(rng.integers(2, 9))
        zt = separated_logits(rng, gamma + 1, V)
        zd = separated_logits(rng, gamma, V)
        g = zt.argmax(axis=1)
        # Draft tokens: mostly the target's argmax, so that long accepted runs occur.
        toks = np.where(rng.random(gamma) < 0.7, g[:gamma], rng.integers(0, V, size=gamma))
        u = rng.random(gamma + 1)
        rs = OC.verify_chain_seq(zt, zd, toks, u, 1e-3)
        rg = OG.verify_chain_greedy_seq(zt, toks)
        if (rs["k"], rs["tokens"]) != (rg["k"], rg["tokens"]):
            return False
    return True


def test_zero_temperature_limit_of_stochastic_verify():
    assert _zero_temperature_agrees()


def _matches_chain_tree_walk(seed=4, trials=300):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        gamma = int(rng.integers(1, 7))
        V = int(rng.integers(1, 5))
        zt = rng.integers(-2, 3, size=(gamma + 1, V)).astype(np.float64)   # many ties
        toks = rng.integers(0, V, size=gamma)
        rg = OG.verify_chain_greedy_seq(zt, toks)
        # Chain-shaped tree: node 0 is the committed context, node i+1 holds draft token i and
        # hangs below node i; node i's logit row is target row i.
        parents = [-1] + list(range(gamma))
        tokens = [0] + [int(x) for x in toks]
        rt = OT.verify_tree_one(zt, parents, tokens)
        if (rg["k"], rg["tokens"]) != (rt["k"], rt["tokens"]) or rg["g"] != rt["g"]:
            return False
    return True


def test_matches_tree_walk_on_chain_shaped_trees():
    assert _matches_chain_tree_walk()


def test_flags_and_fallback():
    z = np.array([[0.0, 2.0, 1.0], [np.nan, 0.0, 3.0], [1.0, 1.0, 0.0]])
    r = OG.verify_chain_greedy_seq(z, [1, 2])
    assert r["status"] == OC.ROW_NONFINITE and r["k"] == 2 and r["tokens"] == [1, 2, 0]
    r = OG.verify_chain_greedy_seq(z, [1, 3])
    assert r["status"] == OC.ROW_NONFINITE | OC.ROW_TOKEN_RANGE
    assert r["k"] == 0 and r["tokens"] == [1]


def test_ties_take_the_lowest_id_and_signed_zero():
    z = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, 0.0]])
    r = OG.verify_chain_greedy_seq(z, [0])
    assert r["g"] == [0, 0] and r["k"] == 1 and r["tokens"] == [0, 0]


MUTATIONS = {
    # accept while the draft differs from the target's choice
    "accept_on_mismatch": lambda z, t: _mutant(z, t, lambda x, g: x != g, 0),
    # substitute the choice of the next position instead of the cut position
    "bonus_off_by_one": lambda z, t: _mutant(z, t, lambda x, g: x == g, 1),
    # ties to the highest token id
    "ties_high": lambda z, t: _mutant(z, t, lambda x, g: x == g, 0, high=True),
}


def _mutant(target, toks, accept, shift, high=False):
    target = np.asarray(target, dtype=np.float64)
    gamma = target.shape[0] - 1
    if high:
        g = [int(len(r) - 1 - np.argmax(r[::-1])) for r in target]
    else:
        g = [int(np.argmax(r)) for r in target]
    k = 0
    while k < gamma and accept(int(toks[k]), g[k]):
        k += 1
    y = g[min(k + shift, gamma)]
    return {"k": k, "tokens": [int(x) for x in toks[:k]] + [y], "g": g, "status": 0}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_fail_a_pin(name, monkeypatch):
    monkeypatch.setattr(OG, "verify_chain_greedy_seq", MUTATIONS[name])
    ok = _zero_temperature_agrees(trials=200) and _matches_chain_tree_walk(trials=200)
    assert not ok, f"mutation {name} went undetected"
