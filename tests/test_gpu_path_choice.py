"""Which kernels each chain call runs, as the library chooses them (no forced path): the
measured gates of the one-workgroup, finish, split and early-exit forms, read back through the
library's kernel timing (sv_trace_*).  Every call is also checked against the oracle."""

import numpy as np
import pytest
import torch

from parity import check_chain
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu

SPLIT = {"chain_sweep", "chain_decide", "chain_residual", "chain_draw"}


def kernels_of(batch, monkeypatch, lazy=False, offset=0):
    monkeypatch.delenv("SPECVERIFY_CHAIN_PATH", raising=False)
    d = BD.chain_to_device(batch)
    tgt, drf = d["target"], d["draft"]
    if offset:
        def shifted(t):
            flat = torch.empty(t.numel() + offset, dtype=t.dtype, device=t.device)
            v = flat[offset:].view(t.shape)
            v.copy_(t)
            return v
        tgt, drf = shifted(tgt), shifted(drf)
    torch.cuda.synchronize()
    BD.trace_start(256)
    try:
        out = BD.sv_verify_chain(tgt, drf, d["draft_tokens"], d["uniforms"], d["temperature"],
                                 lazy=lazy)
        torch.cuda.synchronize()
        names = set(BD.trace_kernels())
    finally:
        BD.trace_stop()
    host = {k: v.cpu().numpy() for k, v in out.items()}
    if not lazy:  # the early-exit forms leave p and q NaN after the cut
        check_chain(batch, host)
    return names


@pytest.mark.parametrize("B,gamma,V,dtype,want", [
    (1, 4, 1000, "f32", {"chain_fused"}),                  # small rows (the B = 1 fp32 workload)
    (1, 7, 32000, "bf16", {"chain_sweep", "chain_finish"}),  # B = 1, V = 32000: sweep + finish
    (8, 4, 70000, "bf16", SPLIT),                          # wide rows, small batch: split
    (64, 4, 70000, "bf16", {"chain_sweep", "chain_finish"}),  # wide rows, 16..128: finish
    (200, 2, 20000, "f32", {"chain_fused"}),               # 192..256 sequences fill the chip
    (300, 2, 20000, "bf16", {"chain_sweep", "chain_finish"}),  # B <= 512, narrow residual rows
    (600, 2, 20000, "bf16", SPLIT),                        # past every one-workgroup gate
])
def test_eager_path_choice(B, gamma, V, dtype, want, monkeypatch):
    b = I.chain_gaussian(60 + B, B, gamma, V, dtype, 2.0, 1.0, 0.9)
    assert kernels_of(b, monkeypatch) == want


def test_unaligned_rows_take_split(monkeypatch):
    b = I.chain_gaussian(61, 1, 4, 1000, "f32", 2.0, 1.0, 1.0)
    assert kernels_of(b, monkeypatch, offset=1) == SPLIT


@pytest.mark.parametrize("B,gamma,V,dtype,want", [
    (64, 3, 8000, "bf16", {"chain_fused"}),                       # below 128 sequences: eager
    (128, 3, 8000, "bf16", {"chain_fused"}),                      # few rows: eager
    (256, 3, 8000, "bf16", {"chain_lazy"}),                       # narrow row pairs: one workgroup
    (128, 3, 70000, "f32", {"chain_stage", "chain_stage_decide", "chain_residual",
                            "chain_draw"}),                       # wide pairs: staged
    (192, 3, 65536, "bf16", {"chain_stage", "chain_stage_decide", "chain_residual",
                             "chain_draw"}),                      # 48 MiB of first pairs: staged
    (128, 3, 40000, "f32", {"chain_sweep", "chain_finish"}),      # below that: eager (finish)
])
def test_early_exit_form_choice(B, gamma, V, dtype, want, monkeypatch):
    b = I.chain_gaussian(62 + B, B, gamma, V, dtype, 2.0, 1.0, 1.0)
    assert kernels_of(b, monkeypatch, lazy=True) == want
