"""GPU parity of sv_chain_acceptance_rates against the oracle (through the C ABI)."""

import numpy as np
import pytest
import torch

from parity import check_acceptance_rates
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu


def run_alpha(batch, offset=0):
    d = BD.chain_to_device(batch)
    t, dr = d["target"], d["draft"]
    if offset:
        def shifted(x):
            flat = torch.empty(x.numel() + offset, dtype=x.dtype, device=x.device)
            v = flat[offset:].view(x.shape)
            v.copy_(x)
            return v
        t, dr = shifted(t), shifted(dr)
    out = BD.sv_chain_acceptance_rates(t, dr, d["temperature"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def test_zipf_b64_workload_mean_alpha():
    b = I.chain_zipf_b64_v128256()
    als = check_acceptance_rates(b, run_alpha(b))
    m = float(np.mean(als))
    print(f"[parity] {b.name} mean alpha {m:.4f}", flush=True)
    assert abs(m - 0.70) < 0.03   # the workload's sigma was calibrated for a mean near 0.7


def test_gauss_b256_workload_full(gauss_b256):
    b, _ = gauss_b256
    out = run_alpha(b)
    als = check_acceptance_rates(b, out)
    print(f"[parity] {b.name} mean alpha {np.mean(als):.4f}", flush=True)
    assert np.all((out["alpha"] >= 0) & (out["alpha"] <= 1.0 + 1e-6))


@pytest.mark.parametrize("name", ["gauss_b1_g4_v1000_f32", "gauss_b1_g7_v32000_bf16"])
def test_small_workloads(name):
    b = I.CHAIN_WORKLOADS[name]()
    check_acceptance_rates(b, run_alpha(b))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 7, 2047, 2048, 2049, 5003])
def test_vocab_edges(dtype, V):
    b = I.chain_gaussian(V + 5, 5, 3, V, dtype, 2.0, 1.0, np.array([0.5, 1.0, 1.7, 0.8, 1.2]))
    check_acceptance_rates(b, run_alpha(b))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned(dtype):
    b = I.chain_gaussian(31, 4, 5, 4100, dtype, 2.0, 1.0, 0.9)
    check_acceptance_rates(b, run_alpha(b, offset=1))


def test_special_rows_and_flags():
    b = I.chain_gaussian(32, 6, 3, 3000, "f32", 2.0, 1.0, 1.0)
    b.draft[0] = b.target[0, :3]                  # p == q: alpha 1
    b.target[1, :, :1500] = -np.inf               # disjoint supports at every position
    b.draft[1, :, 1500:] = -np.inf
    b.target[2, 1, 7] = np.nan                    # position 1 undefined
    b.draft[3, 2, :] = -np.inf                    # position 2 undefined (only -inf)
    b.temperature[4] = 0.0                        # bad temperature: T = 1 and a flag
    b.target[5, 0, 11] = np.inf
    out = run_alpha(b)
    check_acceptance_rates(b, out)
    assert np.allclose(out["alpha"][0], 1.0, rtol=1e-5) and np.all(out["alpha"][1] == 0.0)
    assert np.isnan(out["alpha"][2, 1]) and out["status"][2, 1] == BD.ROW_NONFINITE
    assert np.all(out["status"][4] == BD.ROW_BAD_TEMPERATURE)


def test_gamma_64_and_deterministic():
    b = I.chain_gaussian(33, 2, 64, 2100, "bf16", 2.0, 1.0, 0.7)
    first = run_alpha(b)
    check_acceptance_rates(b, first)
    again = run_alpha(b)
    assert np.array_equal(first["alpha"], again["alpha"], equal_nan=True)


def run_with_rates(batch, offset=0, path=None, monkeypatch=None):
    if path is not None:
        monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", path)
    d = BD.chain_to_device(batch)
    t, dr = d["target"], d["draft"]
    if offset:
        def shifted(x):
            flat = torch.empty(x.numel() + offset, dtype=x.dtype, device=x.device)
            v = flat[offset:].view(x.shape)
            v.copy_(x)
            return v
        t, dr = shifted(t), shifted(dr)
    both = BD.sv_verify_chain(t, dr, d["draft_tokens"], d["uniforms"], d["temperature"],
                              want_rates=True)
    plain = BD.sv_verify_chain(t, dr, d["draft_tokens"], d["uniforms"], d["temperature"])
    alone = BD.sv_chain_acceptance_rates(t, dr, d["temperature"])
    torch.cuda.synchronize()
    host = lambda o: {k: v.cpu().numpy() for k, v in o.items()}
    return host(both), host(plain), host(alone)


def _same(a, b, keys):
    for k in keys:
        assert np.array_equal(a[k], b[k], equal_nan=a[k].dtype.kind == "f"), k


@pytest.mark.parametrize("path", ["finish", "split"])
@pytest.mark.parametrize("dtype,B,gamma,V,offset", [
    ("bf16", 5, 4, 5003 - 3, 0), ("f32", 4, 7, 4100, 0), ("bf16", 3, 5, 9001, 3),
    ("f32", 2, 64, 300, 0)])
def test_verify_with_rates_matches_both_calls(dtype, B, gamma, V, offset, path, monkeypatch):
    """sv_verify_chain_with_rates gives sv_verify_chain's outputs and sv_chain_acceptance_rates'
    alpha bit for bit, and the alpha agrees with the oracle (both chain paths it can take)."""
    b = I.chain_gaussian(50 + gamma, B, gamma, V, dtype, 2.0, 1.0, 0.9)
    both, plain, alone = run_with_rates(b, offset, path, monkeypatch)
    _same(both, plain, ("tokens", "num_accepted", "p", "q", "status"))
    _same(both, alone, ("alpha",))
    check_acceptance_rates(b, {"alpha": both["alpha"]})


def test_verify_with_rates_special_rows():
    b = I.chain_gaussian(61, 6, 4, 3000, "f32", 2.0, 1.0, 1.0)
    b.target[1, 2, 17] = np.nan          # target row 2 of sequence 1: alpha_2 NaN, fallback
    b.draft[2, 0, :] = -np.inf           # a draft row without softmax
    b.temperature[3] = 0.0               # bad temperature: fallback, rates still computed at T = 1
    b.target[4, :, 100:] = -np.inf       # masked logits
    both, plain, alone = run_with_rates(b)
    _same(both, plain, ("tokens", "num_accepted", "p", "q", "status"))
    _same(both, alone, ("alpha",))
    assert np.isnan(both["alpha"][1, 2]) and np.isnan(both["alpha"][2, 0])
    check_acceptance_rates(b, {"alpha": both["alpha"]})


def test_verify_with_rates_full_size():
    """The fp32 B=256 gamma=7 V=152064 workload: the combined call against the two separate ones."""
    b = I.chain_b256_v152064()
    both, plain, alone = run_with_rates(b)
    _same(both, plain, ("tokens", "num_accepted", "p", "q", "status"))
    _same(both, alone, ("alpha",))
