"""HIP graph capture of every entry point.

The library launches kernels only (no allocation, no synchronisation, no memset), so a call can be
captured into a graph, as a serving loop does to remove per-launch host cost.  Each test
allocates inputs, outputs and the workspace first, captures one call, then replays the graph on
new seeded inputs copied into the captured buffers.  An eager call on the same inputs runs between
replays.  Every replay is checked bit for bit against that eager call and against the oracle.
"""

import numpy as np
import pytest
import torch

from parity import (check_acceptance_rates, check_chain, check_chain_greedy, check_kv,
                    check_sample, check_tree)
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu

REPLAY_SEEDS = (101, 102, 103)


def _capture(fn):
    """Warm up on a side stream (default priority), then capture fn into a CUDA/HIP graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _host(d):
    return {k: (None if v is None else v.cpu().numpy()) for k, v in d.items()}


def _load(static, fresh):
    for k, t in static.items():
        if isinstance(t, torch.Tensor):
            t.copy_(fresh[k])
    torch.cuda.synchronize()


def _same(a, b):
    for k in a:
        if a[k] is None:
            continue
        assert np.array_equal(a[k], b[k], equal_nan=np.issubdtype(a[k].dtype, np.floating)), k


@pytest.mark.parametrize("dtype,B,gamma,V,mode", [("bf16", 4, 4, 5000, "plain"),
                                                  ("f32", 3, 6, 4100, "plain"),
                                                  ("bf16", 3, 5, 6000, "rates"),
                                                  ("f32", 5, 6, 4100, "lazy"),
                                                  ("bf16", 4, 5, 6000, "staged")])
def test_graph_chain(dtype, B, gamma, V, mode, monkeypatch):
    rates, lazy = mode == "rates", mode in ("lazy", "staged")
    if lazy:  # an early-exit form at this small batch
        monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", mode)
    dev = torch.device("cuda:0")
    gen = lambda seed: I.chain_gaussian(seed, B, gamma, V, dtype, 2.0, 1.0, 0.8)
    d = BD.chain_to_device(gen(100), dev)
    outs = {"tokens": torch.empty((B, gamma + 1), dtype=torch.int32, device=dev),
            "num_accepted": torch.empty((B,), dtype=torch.int32, device=dev),
            "p": torch.empty((B, gamma), dtype=torch.float32, device=dev),
            "q": torch.empty((B, gamma), dtype=torch.float32, device=dev),
            "status": torch.empty((B,), dtype=torch.int32, device=dev)}
    if rates:
        outs["alpha"] = torch.empty((B, gamma), dtype=torch.float32, device=dev)
        ws = BD.workspace(BD.chain_with_rates_workspace_bytes(B, gamma, V, d["dtype"]), dev)
    else:
        ws = BD.workspace(BD.chain_workspace_bytes(B, gamma, V, d["dtype"]), dev)

    def call():
        BD.sv_verify_chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"],
                           d["temperature"], out_tokens=outs["tokens"],
                           out_num_accepted=outs["num_accepted"], out_p=outs["p"],
                           out_q=outs["q"], out_status=outs["status"],
                           out_alpha=outs.get("alpha"), workspace_buf=ws, lazy=lazy)

    g = _capture(call)
    for seed in REPLAY_SEEDS:
        batch = gen(seed)
        _load(d, BD.chain_to_device(batch, dev))
        g.replay()
        torch.cuda.synchronize()
        got = _host(outs)
        eager = _host(BD.sv_verify_chain(d["target"], d["draft"], d["draft_tokens"],
                                         d["uniforms"], d["temperature"], want_rates=rates,
                                         lazy=lazy))
        torch.cuda.synchronize()
        _same(got, eager)
        check_chain(batch, got, lazy=lazy)
        if rates:
            check_acceptance_rates(batch, {"alpha": got["alpha"]})


def test_graph_tree():
    dev = torch.device("cuda:0")
    gen = lambda seed: I.tree_random(seed, 3, 64, 5000, "bf16", boost=20.0, boost_prob=0.8)
    t = BD.tree_to_device(gen(100), dev)
    n_trees, n_nodes = 3, 64
    outs = {"path": torch.empty((n_trees, n_nodes), dtype=torch.int32, device=dev),
            "tokens": torch.empty((n_trees, n_nodes), dtype=torch.int32, device=dev),
            "num_accepted": torch.empty((n_trees,), dtype=torch.int32, device=dev),
            "node_argmax": torch.empty((n_trees, n_nodes), dtype=torch.int32, device=dev),
            "status": torch.empty((n_trees,), dtype=torch.int32, device=dev)}
    ws = BD.workspace(BD.tree_workspace_bytes(n_trees, n_nodes, 5000, torch.bfloat16), dev)

    def call():
        BD.sv_verify_tree(t["logits"], t["parents"], t["node_tokens"], out_path=outs["path"],
                          out_tokens=outs["tokens"], out_num_accepted=outs["num_accepted"],
                          out_node_argmax=outs["node_argmax"], out_status=outs["status"],
                          workspace_buf=ws)

    g = _capture(call)
    for seed in REPLAY_SEEDS:
        batch = gen(seed)
        _load(t, BD.tree_to_device(batch, dev))
        g.replay()
        torch.cuda.synchronize()
        got = _host(outs)
        eager = _host(BD.sv_verify_tree(t["logits"], t["parents"], t["node_tokens"]))
        torch.cuda.synchronize()
        _same(got, eager)
        check_tree(batch, got)


def test_graph_greedy_sample_alpha():
    dev = torch.device("cuda:0")
    # greedy chain verification
    ggen = lambda seed: I.chain_greedy_planted(seed, 4, 5, 4100, "f32")
    gd = BD.greedy_to_device(ggen(100), dev)
    gout = {"tokens": torch.empty((4, 6), dtype=torch.int32, device=dev),
            "num_accepted": torch.empty((4,), dtype=torch.int32, device=dev),
            "argmax": torch.empty((4, 6), dtype=torch.int32, device=dev),
            "status": torch.empty((4,), dtype=torch.int32, device=dev)}
    gws = BD.workspace(BD.chain_greedy_workspace_bytes(4, 5, 4100, torch.float32), dev)
    # draft-side sampler
    sgen = lambda seed: I.sample_gaussian(seed, 6, 5000, "bf16", 2.0, 0.9)
    sd = BD.sample_to_device(sgen(100), dev)
    sout = {"tokens": torch.empty((6,), dtype=torch.int32, device=dev),
            "prob": torch.empty((6,), dtype=torch.float32, device=dev),
            "status": torch.empty((6,), dtype=torch.int32, device=dev)}
    sws = BD.workspace(BD.sample_workspace_bytes(6, 5000, torch.bfloat16), dev)
    # per-position acceptance rates
    agen = lambda seed: I.chain_gaussian(seed, 3, 4, 5000, "bf16", 2.0, 1.0, 1.0)
    ad = BD.chain_to_device(agen(100), dev)
    aout = {"alpha": torch.empty((3, 4), dtype=torch.float32, device=dev),
            "status": torch.empty((3, 4), dtype=torch.int32, device=dev)}
    aws = BD.workspace(BD.acceptance_rates_workspace_bytes(3, 4, 5000, torch.bfloat16), dev)

    def call():
        BD.sv_verify_chain_greedy(gd["target"], gd["draft_tokens"], out_tokens=gout["tokens"],
                                  out_num_accepted=gout["num_accepted"],
                                  out_argmax=gout["argmax"], out_status=gout["status"],
                                  workspace_buf=gws)
        BD.sv_sample(sd["logits"], sd["temperature"], sd["uniforms"], out_tokens=sout["tokens"],
                     out_prob=sout["prob"], out_status=sout["status"], workspace_buf=sws)
        BD.sv_chain_acceptance_rates(ad["target"], ad["draft"], ad["temperature"],
                                     out_alpha=aout["alpha"], out_status=aout["status"],
                                     workspace_buf=aws)

    g = _capture(call)
    for seed in REPLAY_SEEDS:
        gb, sb, ab = ggen(seed), sgen(seed), agen(seed)
        _load(gd, BD.greedy_to_device(gb, dev))
        _load(sd, BD.sample_to_device(sb, dev))
        _load(ad, BD.chain_to_device(ab, dev))
        g.replay()
        torch.cuda.synchronize()
        got_g, got_s, got_a = _host(gout), _host(sout), _host(aout)
        eg = _host(BD.sv_verify_chain_greedy(gd["target"], gd["draft_tokens"]))
        es = _host(BD.sv_sample(sd["logits"], sd["temperature"], sd["uniforms"]))
        ea = _host(BD.sv_chain_acceptance_rates(ad["target"], ad["draft"], ad["temperature"]))
        torch.cuda.synchronize()
        _same(got_g, eg)
        _same(got_s, es)
        _same(got_a, ea)
        check_chain_greedy(gb, got_g)
        check_sample(sb, got_s)
        check_acceptance_rates(ab, got_a)


def test_graph_kv():
    dev = torch.device("cuda:0")
    gen = lambda seed: I.kv_tree_paths(seed, 3, 16, 4096, dst_rows=12)
    k = BD.kv_to_device(gen(100), dev)
    st = torch.empty((3,), dtype=torch.int32, device=dev)

    def call():
        BD.sv_compact_accepted(k["src"], k["dst"], k["num_accepted"], k["dst_start"], k["path"],
                               out_status=st)

    g = _capture(call)
    for seed in REPLAY_SEEDS:
        batch = gen(seed)
        _load(k, BD.kv_to_device(batch, dev))
        g.replay()
        torch.cuda.synchronize()
        dst_graph, st_graph = k["dst"].cpu().numpy(), st.cpu().numpy()
        k["dst"].copy_(torch.from_numpy(batch.dst_init).to(dev))
        eager = BD.sv_compact_accepted(k["src"], k["dst"], k["num_accepted"], k["dst_start"],
                                       k["path"])["status"]
        torch.cuda.synchronize()
        assert np.array_equal(dst_graph, k["dst"].cpu().numpy())
        assert np.array_equal(st_graph, eager.cpu().numpy())
        check_kv(batch, dst_graph, st_graph)
