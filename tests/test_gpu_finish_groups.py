"""chain_finish with several workgroups per sequence (rows of 16 chunks or more: 4 per sequence up
to 64 sequences, 2 up to 128), through the C ABI.

Each workgroup takes the decision from the sequence's partials and the residual masses of every
G-th chunk; the masses are handed to the last workgroup to arrive, which draws.  Checked bit for
bit against one workgroup per sequence for every step (chain_fused) and against the multi-kernel
path, and against the oracle, on batches holding residual draws, a bonus draw and a fallback row;
the trace confirms the sweep-plus-finish launches ran.  The combined call with acceptance rates
takes the same form.
"""

import numpy as np
import pytest
import torch

from parity import check_acceptance_rates, check_chain
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu

BF16_NAN = 0x7FC0

CASES = [
    (1, 4, 32000, "bf16"),    # 16 chunks, 4 workgroups (the B = 1 bf16 workload's shape)
    (5, 7, 40000, "f32"),     # 20 chunks, 4 workgroups
    (64, 3, 32768, "bf16"),   # the largest batch with 4 workgroups per sequence
    (100, 2, 32000, "bf16"),  # 2 workgroups per sequence
    (128, 3, 36000, "f32"),   # 18 chunks; the largest batch with 2 workgroups
    (64, 4, 70000, "bf16"),   # a 273 KiB row pair: finish by the wide-row gate (16..128 sequences)
]


def batch(B, gamma, V, dtype):
    """Poor drafts (most sequences cut early and draw from the residual); from 3 sequences on,
    sequence 1 drafts the target's own rows (p = q: every draft accepted, the bonus draw) and
    sequence 2 holds a NaN (the fallback result)."""
    b = I.chain_gaussian(300 + B, B, gamma, V, dtype, 2.0, 3.0, np.linspace(0.5, 1.5, B),
                         name=f"finish groups B={B} gamma={gamma} V={V} {dtype}")
    if B >= 3:
        b.draft[1] = b.target[1, :gamma]
        b.target[2, 0, 5] = BF16_NAN if dtype == "bf16" else np.nan
    return b


def call(d, path, monkeypatch, **kw):
    monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", path)
    torch.cuda.synchronize()
    BD.trace_start(256)
    try:
        out = BD.sv_verify_chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"],
                                 d["temperature"], **kw)
        torch.cuda.synchronize()
        names = set(BD.trace_kernels())
    finally:
        BD.trace_stop()
    return {k: v.cpu().numpy() for k, v in out.items()}, names


@pytest.mark.parametrize("B,gamma,V,dtype", CASES)
def test_same_bits_as_one_workgroup_and_oracle(B, gamma, V, dtype, monkeypatch):
    b = batch(B, gamma, V, dtype)
    d = BD.chain_to_device(b)
    outs = {}
    for path in ("finish", "fused", "split"):
        outs[path], names = call(d, path, monkeypatch)
        if path == "finish":
            assert names == {"chain_sweep", "chain_finish"}, names
    counts = check_chain(b, outs["finish"])
    print(f"[parity] {b.name}: {counts}", flush=True)
    fin = outs["finish"]
    if B >= 3:
        assert fin["num_accepted"][1] == gamma, "sequence 1 should accept every draft"
        assert fin["status"][2] & BD.ROW_NONFINITE and fin["num_accepted"][2] == 0
    assert np.any((fin["num_accepted"] < gamma) & (fin["status"] == 0)), "no residual draw"
    for path in ("fused", "split"):
        for k in fin:
            assert np.array_equal(outs[path][k], fin[k], equal_nan=True), (path, k)


def test_wide_rows_take_finish_unforced(monkeypatch):
    b = batch(*CASES[5])
    d = BD.chain_to_device(b)
    monkeypatch.delenv("SPECVERIFY_CHAIN_PATH", raising=False)
    torch.cuda.synchronize()
    BD.trace_start(256)
    try:
        out = BD.sv_verify_chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"],
                                 d["temperature"])
        torch.cuda.synchronize()
        names = set(BD.trace_kernels())
    finally:
        BD.trace_stop()
    assert names == {"chain_sweep", "chain_finish"}, names
    check_chain(b, {k: v.cpu().numpy() for k, v in out.items()})


@pytest.mark.parametrize("B,gamma,V,dtype", [CASES[0], CASES[3], CASES[5]])
def test_with_rates(B, gamma, V, dtype, monkeypatch):
    b = batch(B, gamma, V, dtype)
    d = BD.chain_to_device(b)
    plain, _ = call(d, "finish", monkeypatch)
    rated, names = call(d, "finish", monkeypatch, want_rates=True)
    assert "chain_finish" in names, names
    for k in plain:
        assert np.array_equal(rated[k], plain[k], equal_nan=True), k
    seqs = [s for s in range(B) if not rated["status"][s]]
    check_acceptance_rates(b, {"alpha": rated["alpha"]}, seqs=seqs)


def test_repeated_calls_reuse_the_counts(monkeypatch):
    # The arrival counts live in the workspace and are cleared by each call's sweep: calls in a
    # row on one workspace, with a batch of another size between them, give the same bits.
    b = batch(*CASES[0])
    small = batch(*CASES[3])
    d, ds = BD.chain_to_device(b), BD.chain_to_device(small)
    ws = BD.workspace(BD.chain_workspace_bytes(small.B, small.gamma, small.V, ds["target"].dtype),
                      ds["target"].device)
    first, _ = call(d, "finish", monkeypatch, workspace_buf=ws)
    for _ in range(3):
        call(ds, "finish", monkeypatch, workspace_buf=ws)
        again, _ = call(d, "finish", monkeypatch, workspace_buf=ws)
        for k in first:
            assert np.array_equal(again[k], first[k], equal_nan=True), k
