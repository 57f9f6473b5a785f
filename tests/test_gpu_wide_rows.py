"""GPU parity at row widths far past the workloads', and the one-workgroup forms' LDS budget.

V = 1,000,008 is 488 full chunks of 2048 elements and a ragged tail of 584, so every merge,
chunk search and scan runs over hundreds of partials per row; V = 1,000,003 (odd) also leaves
every row but the first unaligned, which the scalar-load forms take.  The one-workgroup chain
forms keep a sequence's chunk partials in LDS (32 KiB at most); a sequence whose partials do not
fit takes the split path (or, for the early exit, the eager entry point), even when a form is
forced.  Every call is checked against the oracle.
"""

import numpy as np
import pytest
import torch

from parity import (check_acceptance_rates, check_chain, check_chain_greedy, check_sample,
                    check_tree)
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu

WIDE = 1_000_008      # rows 16-byte aligned for fp32 and bf16
WIDE_ODD = 1_000_003  # unaligned rows
SPLIT = {"chain_sweep", "chain_decide", "chain_residual", "chain_draw"}


def traced(fn):
    """Run fn() (a library call) and return (its outputs on the host, the kernels it ran)."""
    torch.cuda.synchronize()
    BD.trace_start(256)
    try:
        out = fn()
        torch.cuda.synchronize()
        names = set(BD.trace_kernels())
    finally:
        BD.trace_stop()
    return {k: v.cpu().numpy() for k, v in out.items()}, names


def chain_call(d, **kw):
    return lambda: BD.sv_verify_chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"],
                                      d["temperature"], **kw)


def report(name, counts):
    print(f"[parity] wide {name}: {counts}", flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_every_path(dtype, monkeypatch):
    """gamma = 1 keeps 3 rows of 489 partials (27 KiB with the residual masses) within the LDS
    budget, so each of the three paths runs as forced; all agree bit for bit and with the
    oracle."""
    b = I.chain_gaussian(71, 2, 1, WIDE, dtype, 2.0, 1.0, 0.9)
    d = BD.chain_to_device(b)
    want = {"fused": {"chain_fused"}, "finish": {"chain_sweep", "chain_finish"}, "split": SPLIT}
    outs = {}
    for path in ("fused", "finish", "split"):
        monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", path)
        outs[path], names = traced(chain_call(d))
        assert names == want[path], (path, names)
    monkeypatch.delenv("SPECVERIFY_CHAIN_PATH")
    report(f"{dtype} B=2 gamma=1", check_chain(b, outs["split"]))
    for path in ("fused", "finish"):
        for k in outs["split"]:
            assert np.array_equal(outs[path][k], outs["split"][k], equal_nan=True), (path, k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_partials_past_lds_take_split(dtype, monkeypatch):
    """gamma = 4: 9 rows of 489 partials (70 KiB) do not fit, so the library's own choice and a
    forced one-workgroup path both run the split kernels."""
    b = I.chain_gaussian(72, 3, 4, WIDE, dtype, 2.0, 0.5, 1.1)
    d = BD.chain_to_device(b)
    monkeypatch.delenv("SPECVERIFY_CHAIN_PATH", raising=False)
    auto, names = traced(chain_call(d))
    assert names == SPLIT
    report(f"{dtype} B=3 gamma=4", check_chain(b, auto))
    for path in ("fused", "finish"):
        monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", path)
        forced, names = traced(chain_call(d))
        assert names == SPLIT, (path, names)
        for k in auto:
            assert np.array_equal(forced[k], auto[k], equal_nan=True), (path, k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_odd_width_takes_split(dtype, monkeypatch):
    """Unaligned rows: the split path's scalar-load kernels, whatever the forced path."""
    b = I.chain_gaussian(81, 2, 1, WIDE_ODD, dtype, 2.0, 1.0, 0.9)
    d = BD.chain_to_device(b)
    outs = {}
    for path in (None, "fused", "finish"):
        if path is None:
            monkeypatch.delenv("SPECVERIFY_CHAIN_PATH", raising=False)
        else:
            monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", path)
        outs[path], names = traced(chain_call(d))
        assert names == SPLIT, (path, names)
    report(f"{dtype} odd width", check_chain(b, outs[None]))
    for path in ("fused", "finish"):
        for k in outs[None]:
            assert np.array_equal(outs[path][k], outs[None][k], equal_nan=True), (path, k)


def test_many_rows_past_lds_take_split(monkeypatch):
    """gamma = 64 at V = 40000: 129 rows of 20 partials (41 KiB) do not fit either."""
    b = I.chain_gaussian(73, 2, 64, 40000, "f32", 2.0, 0.3, 1.0)
    d = BD.chain_to_device(b)
    monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", "fused")
    out, names = traced(chain_call(d))
    assert names == SPLIT
    report("f32 B=2 gamma=64 V=40000", check_chain(b, out))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_with_rates(dtype, monkeypatch):
    """The combined call (finish path at gamma = 1) against the oracle's rates and chain."""
    b = I.chain_gaussian(74, 2, 1, WIDE, dtype, 2.0, 1.0, 0.8)
    d = BD.chain_to_device(b)
    monkeypatch.delenv("SPECVERIFY_CHAIN_PATH", raising=False)
    out, names = traced(chain_call(d, want_rates=True))
    assert "chain_finish" in names or names >= SPLIT, names
    report(f"{dtype} with rates", check_chain(b, out))
    check_acceptance_rates(b, {"alpha": out["alpha"]})


@pytest.mark.parametrize("form", ["lazy", "staged"])
def test_early_exit_forms(form, monkeypatch):
    """Both early-exit forms at V = 1,000,008 (the one-workgroup form's two rows of partials fit),
    against the oracle and the eager entry point on the same buffers."""
    b = I.chain_gaussian(75, 2, 3, WIDE, "bf16", 2.0, 0.4, 1.0)
    d = BD.chain_to_device(b)
    monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", form)
    lazy, names = traced(chain_call(d, lazy=True))
    assert ("chain_lazy" in names) if form == "lazy" else ("chain_stage" in names), names
    report(f"early exit {form}", check_chain(b, lazy, lazy=True))
    monkeypatch.delenv("SPECVERIFY_CHAIN_PATH")
    eager, _ = traced(chain_call(d))
    for key in ("tokens", "num_accepted", "status"):
        assert np.array_equal(lazy[key], eager[key]), key
    k = eager["num_accepted"]
    upto = np.arange(b.gamma)[None, :] <= k[:, None]
    for key in ("p", "q"):
        assert np.array_equal(lazy[key][upto], eager[key][upto], equal_nan=True), key


def test_one_workgroup_early_exit_past_lds_runs_eager(monkeypatch):
    """V = 2,000,000 (977 chunks): the one-workgroup form's two rows of partials exceed the LDS
    budget, so a forced one-workgroup early exit runs the eager entry point."""
    b = I.chain_gaussian(76, 2, 1, 2_000_000, "f32", 2.0, 1.0, 1.0)
    d = BD.chain_to_device(b)
    monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", "lazy")
    out, names = traced(chain_call(d, lazy=True))
    assert "chain_lazy" not in names and "chain_stage" not in names, names
    report("early exit past LDS", check_chain(b, out))


@pytest.mark.parametrize("V", [WIDE, WIDE_ODD])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tree(dtype, V):
    b = I.tree_random(77, 2, 8, V, dtype, boost=20.0, boost_prob=1.0)  # walks go deep
    d = BD.tree_to_device(b)
    out = BD.sv_verify_tree(d["logits"], d["parents"], d["node_tokens"])
    torch.cuda.synchronize()
    ks = check_tree(b, {k: v.cpu().numpy() for k, v in out.items()})
    print(f"[parity] wide tree {dtype} V={V}: accepted {ks}", flush=True)


@pytest.mark.parametrize("V", [WIDE, WIDE_ODD])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_greedy(dtype, V):
    b = I.chain_greedy_planted(78, 4, 3, V, dtype, match_prob=0.6)
    d = BD.greedy_to_device(b)
    out = BD.sv_verify_chain_greedy(d["target"], d["draft_tokens"])
    torch.cuda.synchronize()
    ks = check_chain_greedy(b, {k: v.cpu().numpy() for k, v in out.items()})
    print(f"[parity] wide greedy {dtype} V={V}: accepted {ks}", flush=True)


@pytest.mark.parametrize("V", [WIDE, WIDE_ODD])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sampler(dtype, V):
    b = I.sample_gaussian(79, 3, V, dtype, 2.0, np.array([0.5, 1.0, 1.7], dtype=np.float32))
    d = BD.sample_to_device(b)
    out = BD.sv_sample(d["logits"], d["temperature"], d["uniforms"])
    torch.cuda.synchronize()
    print(f"[parity] wide sampler {dtype} V={V}: "
          f"{check_sample(b, {k: v.cpu().numpy() for k, v in out.items()})}", flush=True)


@pytest.mark.parametrize("V", [WIDE, WIDE_ODD])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_acceptance_rates(dtype, V):
    b = I.chain_gaussian(80, 2, 3, V, dtype, 2.0, 1.0, 0.9)
    d = BD.chain_to_device(b)
    out = BD.sv_chain_acceptance_rates(d["target"], d["draft"], d["temperature"])
    torch.cuda.synchronize()
    check_acceptance_rates(b, {k: v.cpu().numpy() for k, v in out.items()})
