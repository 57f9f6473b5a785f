"""Optional outputs omitted (NULL) on every entry point that has them: the required outputs are
the same as with every output requested, so each kernel that writes an optional output checks
for NULL, fallback rows included."""

import pytest
import torch

from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu


def _same(full, bare, keys):
    torch.cuda.synchronize()
    for k in keys:
        assert torch.equal(torch.nan_to_num(full[k]), torch.nan_to_num(bare[k])), k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_with_rates(dtype):
    b = I.chain_gaussian(22, 5, 4, 3000, dtype, 2.0, 1.0, 0.9)
    b.temperature[1] = 0.0
    d = BD.chain_to_device(b)
    args = (d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["temperature"])
    full = BD.sv_verify_chain(*args, want_rates=True)
    bare = BD.sv_verify_chain(*args, want_rates=True, want_pq=False, want_status=False)
    _same(full, bare, ("tokens", "num_accepted", "alpha"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tree(dtype):
    b = I.tree_random(23, 4, 40, 3000, dtype, boost=20.0, boost_prob=0.8)
    b.parents[1, 5] = 7  # a bad tree takes the fallback
    d = BD.tree_to_device(b)
    args = (d["logits"], d["parents"], d["node_tokens"])
    full = BD.sv_verify_tree(*args)
    bare = BD.sv_verify_tree(*args, want_argmax=False, want_status=False)
    _same(full, bare, ("path", "tokens", "num_accepted"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_greedy(dtype):
    g = I.chain_greedy_planted(24, 5, 4, 3000, dtype)
    g.draft_tokens[0, 1] = 3000  # out of range: fallback
    d = BD.greedy_to_device(g)
    full = BD.sv_verify_chain_greedy(d["target"], d["draft_tokens"])
    bare = BD.sv_verify_chain_greedy(d["target"], d["draft_tokens"], want_argmax=False,
                                     want_status=False)
    _same(full, bare, ("tokens", "num_accepted"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_acceptance_rates_and_sampler(dtype):
    a = I.chain_gaussian(25, 4, 3, 3000, dtype, 2.0, 1.0, 1.0)
    d = BD.chain_to_device(a)
    full = BD.sv_chain_acceptance_rates(d["target"], d["draft"], d["temperature"])
    bare = BD.sv_chain_acceptance_rates(d["target"], d["draft"], d["temperature"],
                                        want_status=False)
    _same(full, bare, ("alpha",))

    s = I.sample_gaussian(26, 9, 3000, dtype, 2.0, 0.8)
    sd = BD.sample_to_device(s)
    full = BD.sv_sample(sd["logits"], sd["temperature"], sd["uniforms"])
    bare = BD.sv_sample(sd["logits"], sd["temperature"], sd["uniforms"], want_prob=False,
                        want_status=False)
    _same(full, bare, ("tokens",))


def test_kv_compaction():
    k = I.kv_chain(27, 6, 4, 4096, dst_rows=12)
    d1, d2 = BD.kv_to_device(k), BD.kv_to_device(k)
    BD.sv_compact_accepted(d1["src"], d1["dst"], d1["num_accepted"], d1["dst_start"], d1["path"])
    BD.sv_compact_accepted(d2["src"], d2["dst"], d2["num_accepted"], d2["dst_start"], d2["path"],
                           want_status=False)
    torch.cuda.synchronize()
    assert torch.equal(d1["dst"], d2["dst"])
