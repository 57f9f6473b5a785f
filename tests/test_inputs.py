"""The seeded input generators: determinism, storage rounding, sampling, workload shapes."""

import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import softmax as sp_softmax

from oracle.chain import softmax_fp64, widen
from rejection_sampling_verify_chain_amd import inputs as I


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    f = np.concatenate([rng.normal(scale=10.0, size=20000),
                        rng.normal(scale=1e-30, size=100)]).astype(np.float32)
    # exact ties between two bf16 neighbours
    f[:8] = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.0 + 2 ** -7,
                      0.0, -0.0, 65504.0, 1e38], dtype=np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(I.bf16_bits(f), ref)
    assert np.array_equal(I.bf16_value(ref), torch.from_numpy(ref.view(np.int16))
                          .view(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("make", [I.chain_b1_v1000, lambda: I.chain_b1_v32000(gamma=5),
                                  lambda: I.chain_zipf(9, 2, 3, 4000, "bf16", 0.75)])
def test_chain_generators_are_deterministic(make):
    a, b = make(), make()
    for f in ("target", "draft", "draft_tokens", "uniforms", "temperature"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_chain_shapes_and_ranges():
    b = I.chain_b1_v32000(gamma=6)
    assert b.target.shape == (1, 7, 32000) and b.draft.shape == (1, 6, 32000)
    assert b.target.dtype == np.uint16 and b.dtype == "bf16"
    assert b.draft_tokens.dtype == np.int32 and np.all((b.draft_tokens >= 0) & (b.draft_tokens < 32000))
    u = b.uniforms.astype(np.float64)
    assert np.all((u >= 0) & (u < 1)) and np.array_equal(u * 2 ** 24, np.round(u * 2 ** 24))
    assert np.all(b.temperature == np.float32(0.8))
    small = I.chain_b1_v1000()
    assert small.target.dtype == np.float32 and small.rows == 9 and small.logit_bytes == 36000


def test_gumbel_draft_tokens_follow_q():
    rng = np.random.default_rng(1)
    z = rng.normal(size=6).astype(np.float32)
    T = 0.7
    rows = np.repeat(z[None, :], 60000, axis=0)
    toks = I.draft_tokens_gumbel(np.random.SeedSequence(5), rows, np.full(60000, T, np.float32))
    obs = np.bincount(toks, minlength=6)
    assert stats.chisquare(obs, sp_softmax(z.astype(np.float64) / T) * 60000).pvalue > 1e-3


def test_tree_generator_structure():
    t = I.tree_random(3, 8, 64, 500, "bf16")
    assert t.logits.shape == (8, 64, 500)
    for k in range(t.n_trees):
        par, tok = t.parents[k], t.node_tokens[k]
        assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, 64))
        depth = [0] * 64
        for i in range(1, 64):
            depth[i] = depth[par[i]] + 1
        assert max(depth) <= 8
        for u in range(64):
            kids = np.flatnonzero(par == u)
            assert len(kids) <= 4
            assert len(set(tok[kids].tolist())) == len(kids)


def test_tree_boost_lands_on_a_child_token():
    t = I.tree_random(4, 4, 64, 300, "f32", sigma=1.0, boost=50.0, boost_prob=1.0)
    for k in range(t.n_trees):
        for u in range(64):
            kids = np.flatnonzero(t.parents[k] == u)
            if len(kids):
                assert int(np.argmax(t.logits[k, u])) in set(t.node_tokens[k, kids].tolist())


def test_tree_16x64_v32000_deterministic():
    a, b = I.tree_16x64_v32000(), I.tree_16x64_v32000()
    assert np.array_equal(a.logits, b.logits) and np.array_equal(a.parents, b.parents)
    assert a.logits.shape == (16, 64, 32000) and a.logit_bytes == 65536000


def test_zipf_alpha_near_target():
    # mean alpha = sum_x min(p, q) of the calibrated Zipf workload on an independent draw
    b = I.chain_zipf(777, 4, 4, 128256, "bf16", I.ZIPF_DRAFT_SIGMA)
    vals = []
    for s in range(b.B):
        for i in range(b.gamma):
            p = softmax_fp64(widen(b.target[s, i], "bf16"), 1.0)
            q = softmax_fp64(widen(b.draft[s, i], "bf16"), 1.0)
            vals.append(np.minimum(p, q).sum())
    assert abs(np.mean(vals) - 0.7) < 0.03


def test_random_tree_rejects_unreachable_shapes():
    g = np.random.default_rng(0)
    with pytest.raises(ValueError):
        I.random_tree(g, 74, 4096, max_branch=4, max_depth=2)   # at most 1 + 4 + 16 nodes
    with pytest.raises(ValueError):
        I.random_tree(g, 5, 1, max_branch=4, max_depth=3)      # one token: a chain of 4 at most
    parents, tokens = I.random_tree(g, 21, 4096, max_branch=4, max_depth=8)
    assert len(parents) == 21 and parents[0] == -1
