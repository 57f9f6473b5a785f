"""The chain entry point that allocates nothing (sv_verify_chain_noalloc), through the C ABI.

It runs the kernels of sv_verify_chain on the library's static device scratch, so its outputs
must equal sv_verify_chain's bit for bit on the same inputs.  Checked on two calls in a row, the
second with a smaller input (the scratch keeps the first call's contents), on each chain path,
on the largest chain workload, after calls of other shapes, and against the oracle.  The
binding passes caller-owned outputs only; the call itself creates no tensor.  Shapes beyond the
scratch are refused on the host (SV_ERR_SCRATCH, tests/test_abi.py, no GPU needed).
"""

import numpy as np
import pytest
import torch

from parity import check_chain
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu


def outputs(B, gamma, dev):
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    return {"out_tokens": torch.full((B, gamma + 1), -7, **i32),
            "out_num_accepted": torch.full((B,), -7, **i32),
            "out_p": torch.full((B, gamma), -7.0, **f32),
            "out_q": torch.full((B, gamma), -7.0, **f32),
            "out_status": torch.full((B,), -7, **i32)}


def both(batch):
    """(sv_verify_chain outputs, sv_verify_chain_noalloc outputs) as numpy, same device inputs."""
    d = BD.chain_to_device(batch)
    args = (d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["temperature"])
    ref = BD.sv_verify_chain(*args)
    outs = outputs(batch.B, batch.gamma, d["target"].device)
    got = BD.sv_verify_chain_noalloc(*args, **outs)
    torch.cuda.synchronize()
    return ({k: v.cpu().numpy() for k, v in ref.items()},
            {k: v.cpu().numpy() for k, v in got.items()})


def assert_same(ref, got):
    for k in ("tokens", "num_accepted", "p", "q", "status"):
        assert np.array_equal(ref[k], got[k], equal_nan=True), k


@pytest.mark.parametrize("path", ["auto", "fused", "finish", "split"])
def test_two_calls_second_smaller(path, monkeypatch):
    if path != "auto":
        monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", path)
    first = I.chain_gaussian(51, 40, 6, 20000, "bf16", 2.0, 1.0, np.linspace(0.5, 1.5, 40))
    second = I.chain_gaussian(52, 3, 2, 1500, "f32", 2.0, 0.7, 0.9)
    for b in (first, second):
        ref, got = both(b)
        assert_same(ref, got)
        check_chain(b, got)


def test_largest_chain_workload(gauss_b256):
    b, refs = gauss_b256
    ref, got = both(b)
    assert_same(ref, got)
    check_chain(b, got, refs=refs)


def test_after_other_shapes_and_optional_outputs():
    # A large call leaves the scratch full of its partials; later smaller calls of other shapes
    # (and one without the optional outputs) must not read any of it.
    for seed, B, g, V, dt in ((61, 200, 7, 30000, "f32"), (62, 9, 4, 5003, "bf16"),
                              (63, 1, 1, 1, "f32"), (64, 17, 3, 2049, "bf16")):
        b = I.chain_gaussian(seed, B, g, V, dt, 2.0, 1.0, 1.0)
        ref, got = both(b)
        assert_same(ref, got)
    b = I.chain_gaussian(65, 12, 5, 7000, "f32", 2.0, 1.0, 0.8)
    d = BD.chain_to_device(b)
    args = (d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["temperature"])
    outs = outputs(b.B, b.gamma, d["target"].device)
    bare = BD.sv_verify_chain_noalloc(*args, out_tokens=outs["out_tokens"],
                                      out_num_accepted=outs["out_num_accepted"])
    ref = BD.sv_verify_chain(*args)
    torch.cuda.synchronize()
    assert torch.equal(bare["tokens"], ref["tokens"])
    assert torch.equal(bare["num_accepted"], ref["num_accepted"])
