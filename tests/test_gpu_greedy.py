"""GPU parity of sv_verify_chain_greedy against the oracle (through the C ABI)."""

import json
import os

import numpy as np
import pytest
import torch

from parity import check_chain_greedy
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_greedy(batch, offset=0):
    d = BD.greedy_to_device(batch)
    target = d["target"]
    if offset:
        flat = torch.empty(target.numel() + offset, dtype=target.dtype, device=target.device)
        v = flat[offset:].view(target.shape)
        v.copy_(target)
        target = v
    out = BD.sv_verify_chain_greedy(target, d["draft_tokens"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("name", sorted(I.GREEDY_WORKLOADS))
def test_full_size_workloads(name):
    b = I.GREEDY_WORKLOADS[name]()
    ks = check_chain_greedy(b, run_greedy(b))
    print(f"[parity] {name}: mean accepted {np.mean(ks):.2f}, all-accepted {ks.count(b.gamma)}",
          flush=True)
    assert 0 < np.mean(ks) < b.gamma


def test_stochastic_workload_tokens():
    # Draft tokens sampled from q (the stochastic workload at V=32000): mostly early cuts.
    c = I.chain_b1_v32000(gamma=7)
    b = I.GreedyBatch("c2_g7", c.dtype, c.target, c.draft_tokens)
    check_chain_greedy(b, run_greedy(b))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,gamma", [(1, 3), (2, 1), (7, 4), (2047, 5), (2048, 7), (2049, 2),
                                     (5003, 64), (32000, 4)])
def test_integer_logits_with_ties(dtype, V, gamma):
    rng = np.random.default_rng(V * 13 + gamma)
    B = 11
    z = rng.integers(-3, 3, size=(B, gamma + 1, V)).astype(np.float32)
    plant = rng.integers(0, V, size=(B, gamma + 1))
    for bb in range(B):
        for i in range(gamma + 1):
            if rng.random() < 0.85:
                z[bb, i, plant[bb, i]] = 4.0
    toks = np.where(rng.random((B, gamma)) < 0.8, plant[:, :gamma],
                    rng.integers(0, V, size=(B, gamma))).astype(np.int32)
    b = I.GreedyBatch(f"ties_{V}_{gamma}", dtype, I.bf16_bits(z) if dtype == "bf16" else z, toks)
    check_chain_greedy(b, run_greedy(b))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_rows(dtype):
    b = I.chain_greedy_planted(21, 5, 6, 4100, dtype)
    check_chain_greedy(b, run_greedy(b, offset=1))


def test_nan_rows_and_bad_tokens():
    b = I.chain_greedy_planted(22, 6, 4, 3000, "f32")
    b.target[1, 2, 17] = np.nan                  # NaN in a row: flagged, skipped by the argmax
    b.target[2, 0, :] = np.nan                   # a row of only NaN: argmax 0
    b.draft_tokens[3, 1] = 3000                  # out of range: fallback [g_0]
    b.draft_tokens[4, 0] = -1
    b.target[5, :, :] = -np.inf                  # only -inf: argmax 0 everywhere
    out = run_greedy(b)
    check_chain_greedy(b, out)
    assert out["status"][1] == BD.ROW_NONFINITE and out["status"][3] == BD.ROW_TOKEN_RANGE


def test_golden_greedy_example():
    g = json.load(open(os.path.join(GOLDEN, "p2_greedy_example.json")))
    t = g["tree"]
    V = len(g["vocab"])
    z = np.zeros((1, len(t["target_choice_per_node"]), V), dtype=np.float32)
    for i, c in enumerate(t["target_choice_per_node"]):
        z[0, i, c] = 5.0
    b = I.GreedyBatch("golden", "f32", z, np.array([t["node_tokens"][1:]], dtype=np.int32))
    out = run_greedy(b)
    check_chain_greedy(b, out)
    assert out["num_accepted"][0] == g["expected"]["num_accepted"]
    assert list(out["tokens"][0][:3]) == g["expected"]["tokens"]


def test_deterministic():
    b = I.chain_greedy_planted(23, 32, 5, 20000, "bf16")
    first = run_greedy(b)
    for _ in range(3):
        again = run_greedy(b)
        for k in first:
            assert np.array_equal(first[k], again[k])


def test_two_chunks_per_wave_odd_chunk_count():
    # 61 sequences x 5 target rows x 33 chunks (V = 66000) = 10065 chunks: more than one round of
    # resident waves at one chunk per wave and at most one at two, so the argmax takes two chunks
    # per wave, and the last wave holds a single chunk.  Ties, signed zeros and NaN sit in the
    # second chunk of a wave's pair and across the pair's boundary.
    B, gamma, V = 61, 4, 66000
    rng = np.random.default_rng(77)
    z = rng.normal(scale=2.0, size=(B, gamma + 1, V)).astype(np.float32)
    rows = z.reshape(-1, V)
    for r in range(0, rows.shape[0], 7):
        rows[r, [4096 + 17, 6144 + 3, 2047]] = 30.0            # ties across chunks 1..3
    for r in range(3, rows.shape[0], 11):
        rows[r, :] = -1.0
        rows[r, 2048 + 5], rows[r, 2048 + 1] = -0.0, 0.0        # both zeros in the second chunk
    rows[5, 2049] = np.nan                                     # NaN flagged, never the maximum
    rows[rows.shape[0] - 1, V - 1] = 40.0                      # maximum in the lone last chunk
    plant = np.argmax(z, axis=2)
    toks = np.where(rng.random((B, gamma)) < 0.7, plant[:, :gamma],
                    rng.integers(0, V, size=(B, gamma))).astype(np.int32)
    b = I.GreedyBatch("two_chunks", "f32", z, toks)
    out = run_greedy(b)
    check_chain_greedy(b, out)
    bb = I.GreedyBatch("two_chunks_bf16", "bf16", I.bf16_bits(z), toks)
    check_chain_greedy(bb, run_greedy(bb))
