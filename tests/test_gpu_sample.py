"""GPU parity of sv_sample against the oracle (through the C ABI)."""

import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import softmax as sp_softmax

from parity import assert_band_limit, check_sample
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu


def run_sample(batch, offset=0):
    d = BD.sample_to_device(batch)
    z = d["logits"]
    if offset:
        flat = torch.empty(z.numel() + offset, dtype=z.dtype, device=z.device)
        v = flat[offset:].view(z.shape)
        v.copy_(z)
        z = v
    out = BD.sv_sample(z, d["temperature"], d["uniforms"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("name", sorted(I.SAMPLE_WORKLOADS))
def test_full_size_workloads(name):
    b = I.SAMPLE_WORKLOADS[name]()
    c = check_sample(b, run_sample(b))
    print(f"[parity] {name}: {c}", flush=True)
    assert_band_limit(name, c)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 7, 63, 64, 65, 2047, 2048, 2049, 5003, 32000])
def test_vocab_edges(dtype, V):
    b = I.sample_gaussian(V + 1, 40, V, dtype, 2.0, np.linspace(0.3, 2.0, 40))
    check_sample(b, run_sample(b))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned(dtype):
    b = I.sample_gaussian(41, 17, 4100, dtype, 2.0, 0.9)
    check_sample(b, run_sample(b, offset=1))


def test_masked_tokens_extremes_and_flags():
    b = I.sample_gaussian(42, 12, 3000, "f32", 2.0, 1.0)
    b.logits[0, ::2] = -np.inf                       # masked tokens are never drawn
    b.uniforms[1] = 0.0
    b.uniforms[2] = np.float32(1 - 2 ** -24)
    b.temperature[3] = 1e-30                         # effectively greedy: the argmax
    b.temperature[4] = 50.0
    b.logits[5, 9] = np.nan
    b.temperature[6] = -1.0
    b.uniforms[7] = 1.0
    b.logits[8, :] = -np.inf
    out = run_sample(b)
    check_sample(b, out)
    assert out["tokens"][0] % 2 == 1
    assert out["tokens"][3] == int(np.argmax(b.logits[3]))
    assert out["status"][5] == BD.ROW_NONFINITE and out["status"][6] == BD.ROW_BAD_TEMPERATURE
    assert out["status"][7] == BD.ROW_BAD_UNIFORM and out["status"][8] == BD.ROW_NONFINITE


def test_distribution_on_gpu():
    # Many rows with the same logits and fresh uniforms: the GPU draws follow softmax(z / T).
    V, rows, T = 20, 40000, 0.7
    rng = np.random.default_rng(43)
    z = rng.normal(0, 1.5, size=V).astype(np.float32)
    b = I.SampleBatch("dist", "f32", np.tile(z, (rows, 1)), np.full(rows, T, np.float32),
                      (rng.integers(0, 1 << 24, rows) / float(1 << 24)).astype(np.float32))
    out = run_sample(b)
    obs = np.bincount(out["tokens"], minlength=V)
    assert stats.chisquare(obs, sp_softmax(z.astype(np.float64) / T) * rows).pvalue > 1e-3


def test_deterministic():
    b = I.sample_gaussian(44, 64, 20000, "bf16", 2.0, 0.8)
    first = run_sample(b)
    again = run_sample(b)
    for k in first:
        assert np.array_equal(first[k], again[k], equal_nan=True)
