"""GPU parity on seeded random shapes, for every entry point.

Each case draws its shape (batch, gamma, vocabulary, node count, row width), dtype, temperature
and logit scales from a fixed seed, builds the inputs with the seeded generators, and compares
the library's outputs with the oracle by the same rules as the other parity tests.  The shapes
cross the chunk (2048) and vector-width boundaries at random, including V = 1 and gamma = 1;
chain cases run on all three chain paths and on both early-exit forms.
"""

import numpy as np
import pytest
import torch

from parity import (check_acceptance_rates, check_chain, check_chain_greedy, check_kv,
                    check_sample, check_tree)
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu

CASES = range(12)


def _rng(kind, case):
    return np.random.default_rng([7919, kind, case])


def _vocab(rng):
    return int(rng.choice([1, 2, 3, 8, 63, 1000, 2047, 2048, 2049, 4096, 5003, 8192, 9001]))


def _host(out):
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in out.items()}


@pytest.mark.parametrize("path", ["fused", "finish", "split", "lazy", "staged"])
@pytest.mark.parametrize("case", CASES)
def test_random_chain(case, path, monkeypatch):
    rng = _rng(1, case)
    B, gamma, V = int(rng.integers(1, 24)), int(rng.integers(1, 13)), _vocab(rng)
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    T = rng.uniform(0.3, 2.0, size=B).astype(np.float32)
    b = I.chain_gaussian(1000 + case, B, gamma, V, dtype, float(rng.uniform(0.5, 4.0)),
                         float(rng.uniform(0.1, 2.0)), T, draft_scale=float(rng.uniform(0.5, 1.0)))
    monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", path)
    d = BD.chain_to_device(b)
    lazy = path in ("lazy", "staged")  # the early-exit entry point, forced onto either form
    check_chain(b, _host(BD.sv_verify_chain(d["target"], d["draft"], d["draft_tokens"],
                                            d["uniforms"], d["temperature"], lazy=lazy)),
                lazy=lazy)


@pytest.mark.parametrize("case", CASES)
def test_random_chain_with_rates(case):
    rng = _rng(2, case)
    B, gamma, V = int(rng.integers(1, 12)), int(rng.integers(1, 9)), _vocab(rng)
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    b = I.chain_gaussian(2000 + case, B, gamma, V, dtype, float(rng.uniform(0.5, 4.0)),
                         float(rng.uniform(0.1, 2.0)), float(rng.uniform(0.3, 2.0)))
    d = BD.chain_to_device(b)
    out = _host(BD.sv_verify_chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"],
                                   d["temperature"], want_rates=True))
    check_chain(b, out)
    check_acceptance_rates(b, {"alpha": out["alpha"]})


@pytest.mark.parametrize("case", CASES)
def test_random_tree(case):
    rng = _rng(3, case)
    n_trees, n_nodes, V = int(rng.integers(1, 9)), int(rng.integers(1, 140)), _vocab(rng)
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    b = I.tree_random(3000 + case, n_trees, n_nodes, V, dtype, boost=float(rng.uniform(0, 20)),
                      boost_prob=float(rng.uniform(0, 1)), max_branch=min(4, V),
                      max_depth=n_nodes)
    d = BD.tree_to_device(b)
    check_tree(b, _host(BD.sv_verify_tree(d["logits"], d["parents"], d["node_tokens"])))


@pytest.mark.parametrize("case", CASES)
def test_random_greedy_sample_alpha(case):
    rng = _rng(4, case)
    B, gamma, V = int(rng.integers(1, 20)), int(rng.integers(1, 13)), _vocab(rng)
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    g = I.chain_greedy_planted(4000 + case, B, gamma, V, dtype,
                               match_prob=float(rng.uniform(0, 1)))
    gd = BD.greedy_to_device(g)
    check_chain_greedy(g, _host(BD.sv_verify_chain_greedy(gd["target"], gd["draft_tokens"])))

    rows = int(rng.integers(1, 40))
    s = I.sample_gaussian(5000 + case, rows, V, dtype, float(rng.uniform(0.5, 4.0)),
                          rng.uniform(0.3, 2.0, size=rows).astype(np.float32))
    sd = BD.sample_to_device(s)
    check_sample(s, _host(BD.sv_sample(sd["logits"], sd["temperature"], sd["uniforms"])))

    a = I.chain_gaussian(6000 + case, B, gamma, V, dtype, float(rng.uniform(0.5, 4.0)),
                         float(rng.uniform(0.1, 2.0)), float(rng.uniform(0.3, 2.0)))
    ad = BD.chain_to_device(a)
    check_acceptance_rates(a, _host(BD.sv_chain_acceptance_rates(ad["target"], ad["draft"],
                                                                 ad["temperature"])))


@pytest.mark.parametrize("case", CASES)
def test_random_kv(case):
    rng = _rng(5, case)
    row_bytes = int(rng.choice([4, 16, 48, 256, 4096, 6000, 65536]))
    if rng.random() < 0.5:
        k = I.kv_tree_paths(7000 + case, int(rng.integers(1, 6)), int(rng.integers(1, 40)),
                            row_bytes, dst_rows=int(rng.integers(8, 40)))
    else:
        k = I.kv_chain(7000 + case, int(rng.integers(1, 10)), int(rng.integers(1, 9)), row_bytes,
                       dst_rows=int(rng.integers(10, 40)))
    kd = BD.kv_to_device(k)
    st = BD.sv_compact_accepted(kd["src"], kd["dst"], kd["num_accepted"], kd["dst_start"],
                                kd["path"])["status"]
    torch.cuda.synchronize()
    check_kv(k, kd["dst"].cpu().numpy(), st.cpu().numpy())
