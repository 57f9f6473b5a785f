"""GPU parity of sv_verify_chain against the oracle (through the C ABI)."""

import json
import os

import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import softmax as sp_softmax

from parity import assert_band_limit, check_chain
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True, params=["fused", "finish", "split"])
def chain_path(request, monkeypatch):
    """Every test runs on the three chain paths: one workgroup per sequence for every step, the
    sweep followed by one workgroup per sequence for the rest (both forced wherever their LDS image
    fits; rows that are not 16-byte aligned always take the multi-kernel path), and the
    multi-kernel path."""
    monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", request.param)
    return request.param


def run_chain(batch, offset=0):
    """Run the library on a ChainBatch; offset > 0 shifts the logit base pointers by that many
    elements (an unaligned view of a larger buffer)."""
    d = BD.chain_to_device(batch)
    tgt, drf = d["target"], d["draft"]
    if offset:
        def shifted(t):
            flat = torch.empty(t.numel() + offset, dtype=t.dtype, device=t.device)
            v = flat[offset:].view(t.shape)
            v.copy_(t)
            return v
        tgt, drf = shifted(tgt), shifted(drf)
    out = BD.sv_verify_chain(tgt, drf, d["draft_tokens"], d["uniforms"], d["temperature"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def report(name, counts):
    print(f"[parity] {name}: {counts}", flush=True)


def test_gauss_b1_g4_v1000_f32():
    b = I.chain_b1_v1000()
    report(b.name, check_chain(b, run_chain(b)))


@pytest.mark.parametrize("gamma", [4, 5, 6, 7])
def test_gauss_b1_v32000_bf16(gamma):
    b = I.chain_b1_v32000(gamma=gamma)
    report(b.name, check_chain(b, run_chain(b)))


def test_zipf_b64_g4_v128256_full():
    b = I.chain_zipf_b64_v128256()
    counts = check_chain(b, run_chain(b))
    report(b.name, counts)
    assert_band_limit(b.name, counts)


def test_gauss_b256_g7_v152064_full(gauss_b256):
    # Full workload, every sequence against the oracle, on each chain path (the benchmark's own
    # launch is the path the library picks here: one workgroup per sequence).
    b, refs = gauss_b256
    out = run_chain(b)
    counts = check_chain(b, out, refs=refs)
    report(b.name, counts)
    assert_band_limit(b.name, counts)
    assert counts["fallback"] == 0
    assert counts["exact"] + counts["accept_band"] + counts["edge_band"] == 256
    k = out["num_accepted"]
    assert np.all((k >= 0) & (k <= 7))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_large_batch(dtype):
    # 8192 sequences: grids of many workgroups on every path (the batch is past every
    # one-workgroup gate, so the automatic choice would be the multi-kernel path); every
    # sequence against the oracle.
    b = I.chain_gaussian(29, 8192, 2, 64, dtype, 2.0, 1.0, np.linspace(0.3, 2.0, 8192))
    counts = check_chain(b, run_chain(b))
    report(f"large batch {dtype}", counts)
    assert counts["fallback"] == 0
    assert counts["exact"] + counts["accept_band"] + counts["edge_band"] == 8192


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 7, 63, 64, 65, 1000, 2047, 2048, 2049, 4100, 5003, 8191])
def test_edge_shapes(dtype, V):
    for B, gamma, T in ((1, 1, 1.0), (3, 2, 0.5), (17, 7, 2.0)):
        b = I.chain_gaussian(V * 31 + B, B, gamma, V, dtype, 2.0, 1.0, T)
        report(f"gauss {dtype} V={V} B={B} g={gamma}", check_chain(b, run_chain(b)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_base_pointer(dtype):
    b = I.chain_gaussian(5, 4, 3, 4096, dtype, 2.0, 1.0, 1.0)
    report(f"unaligned {dtype}", check_chain(b, run_chain(b, offset=1)))


def test_gamma_max_and_all_accept():
    # draft == target: every token is accepted; gamma = 64 exercises the full-wave mask.
    rng = np.random.default_rng(0)
    t = rng.normal(scale=2.0, size=(2, 65, 300)).astype(np.float32)
    b = I.chain_from_logits(6, t, t[:, :64], 0.9)
    out = run_chain(b)
    assert np.all(out["num_accepted"] == 64)
    report("gamma=64 p==q", check_chain(b, out))


def test_masked_logits_and_disjoint_support():
    rng = np.random.default_rng(1)
    B, g, V = 6, 3, 3000
    t = rng.normal(scale=2.0, size=(B, g + 1, V)).astype(np.float32)
    d = (t[:, :g] + rng.normal(size=(B, g, V))).astype(np.float32)
    t[rng.random(t.shape) < 0.3] = -np.inf
    d[rng.random(d.shape) < 0.3] = -np.inf
    d[0, 0, :1500] = -np.inf  # disjoint supports at sequence 0, position 0
    t[0, 0, 1500:] = -np.inf
    b = I.chain_from_logits(7, t, d, 1.0)
    out = run_chain(b)
    assert out["num_accepted"][0] == 0 and out["tokens"][0, 0] < 1500
    report("masked", check_chain(b, out))


def test_data_errors_set_flags():
    b = I.chain_gaussian(8, 6, 3, 500, "f32", 2.0, 1.0, 1.0)
    b.draft_tokens[0, 1] = 500
    b.target[1, 2, 17] = np.nan
    b.draft[2, 0, :] = -np.inf
    b.temperature[3] = 0.0
    b.uniforms[4, 3] = 1.0
    b.target[5, 0, 3] = np.inf
    out = run_chain(b)
    want = [BD.ROW_TOKEN_RANGE, BD.ROW_NONFINITE, BD.ROW_NONFINITE, BD.ROW_BAD_TEMPERATURE,
            BD.ROW_BAD_UNIFORM, BD.ROW_NONFINITE]
    assert list(out["status"]) == want
    assert np.all(out["num_accepted"] == 0) and np.all(out["tokens"][:, 0] == 0)
    report("data errors", check_chain(b, out))


def test_golden_sequence_diagram():
    g = json.load(open(os.path.join(GOLDEN, "p1_sequence_diagram.json")))
    s = g["scripted"]
    t = np.log(np.array(s["target_probs"], dtype=np.float32))[None]
    d = np.log(np.array(s["draft_probs"], dtype=np.float32))[None]
    b = I.chain_from_logits(0, t, d, s["temperature"])
    b.draft_tokens[0] = s["draft_tokens"]
    b.uniforms[0] = s["uniforms"]
    out = run_chain(b)
    assert int(out["num_accepted"][0]) == g["expected"]["num_accepted"]
    assert list(out["tokens"][0, :3]) == g["expected"]["tokens"]


def test_deterministic():
    b = I.chain_b1_v32000(gamma=7)
    o1, o2 = run_chain(b), run_chain(b)
    for k in o1:
        assert np.array_equal(o1[k], o2[k]), k


def test_same_bits_on_another_stream():
    # No float atomics and no cross-call state: a call on a side stream gives the same bits.
    b = I.chain_gaussian(17, 6, 5, 5003, "bf16", 2.0, 1.0, 0.9)
    d = BD.chain_to_device(b)
    args = (d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["temperature"])
    ref = BD.sv_verify_chain(*args)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = BD.sv_verify_chain(*args, stream=side)
    side.synchronize()
    for k in ref:
        assert torch.equal(torch.nan_to_num(ref[k]), torch.nan_to_num(got[k])), k


def _many(zt, zd, T, N, seed):
    """N sequences sharing the logits, with draft tokens drawn from q and fresh uniforms."""
    rng = np.random.default_rng(seed)
    g, V = zd.shape
    t = np.broadcast_to(zt.astype(np.float32), (N, g + 1, V)).copy()
    d = np.broadcast_to(zd.astype(np.float32), (N, g, V)).copy()
    b = I.chain_from_logits(seed, t, d, T)
    return b


def test_theorem1_on_gpu_outputs():
    rng = np.random.default_rng(2)
    V, g, T = 6, 3, 0.8
    zt = rng.normal(size=(g + 1, V))
    zd = zt[:g] + rng.normal(size=(g, V))
    b = _many(zt, zd, T, 200000, 3)
    out = run_chain(b)
    ks, toks = out["num_accepted"], out["tokens"]
    zt32 = zt.astype(np.float32).astype(np.float64)
    for j in range(g + 1):
        sel = ks >= j
        obs = np.bincount(toks[sel, j], minlength=V)
        pv = stats.chisquare(obs, sp_softmax(zt32[j] / T) * sel.sum()).pvalue
        assert pv > 1e-3, (j, pv)


def test_closed_form_on_gpu_outputs():
    g, a, bq = 5, 0.6, 0.3
    alpha = 1 - abs(a - bq)
    zt = np.log(np.array([[a, 1 - a]] * (g + 1)))
    zd = np.log(np.array([[bq, 1 - bq]] * g))
    b = _many(zt, zd, 1.0, 200000, 4)
    ks = run_chain(b)["num_accepted"].astype(np.int64)
    emitted = ks + 1
    expect = (1 - alpha ** (g + 1)) / (1 - alpha)
    se = emitted.std(ddof=1) / np.sqrt(len(emitted))
    assert abs(emitted.mean() - expect) < 4 * se
    probs = np.array([alpha ** k * (1 - alpha) for k in range(g)] + [alpha ** g])
    assert stats.chisquare(np.bincount(ks, minlength=g + 1), probs * len(ks)).pvalue > 1e-3


@pytest.mark.parametrize("T", [1e-30, 1.4e-45, 1e-3, 50.0, 1e30])
def test_extreme_temperatures(T):
    b = I.chain_gaussian(9, 5, 4, 777, "f32", 2.0, 1.0, T)
    report(f"T={T}", check_chain(b, run_chain(b)))


@pytest.mark.parametrize("dtype,B,gamma,V,T", [("bf16", 3, 7, 32000, 0.8), ("f32", 5, 4, 5003, 1.0),
                                                ("bf16", 2, 64, 300, 1.3)])
def test_paths_bit_identical(dtype, B, gamma, V, T, monkeypatch):
    """The three paths compute every step with the same device functions: all outputs agree bit
    for bit (p and q included), on sequences that cut early, accept everything, and fall back."""
    b = I.chain_gaussian(31, B, gamma, V, dtype, 2.0, 1.0, T)
    b.temperature[0] = -1.0  # a fallback sequence
    outs = {}
    for path in ("fused", "finish", "split"):
        monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", path)
        outs[path] = run_chain(b)
    for k in outs["split"]:
        for path in ("fused", "finish"):
            assert np.array_equal(outs[path][k], outs["split"][k], equal_nan=True), (path, k)


def test_concurrent_host_threads():
    # The library keeps no per-call host state: calls from several host threads, each on its
    # own stream, give the same bits as one call at a time.
    import threading
    batches = [I.chain_gaussian(40 + t, 5, 4, 3000 + 100 * t, "f32", 2.0, 1.0, 1.0)
               for t in range(4)]
    devs = [BD.chain_to_device(b) for b in batches]
    refs = []
    for d in devs:
        refs.append(BD.sv_verify_chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"],
                                       d["temperature"]))
    torch.cuda.synchronize()
    got = [None] * len(devs)
    errors = []

    def work(t):
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.default_stream())
            d = devs[t]
            # Outputs and workspace are allocated on the thread's stream too, so the caching
            # allocator hands a freed block only to later work on that same stream.
            with torch.cuda.stream(s):
                for _ in range(20):
                    o = BD.sv_verify_chain(d["target"], d["draft"], d["draft_tokens"],
                                           d["uniforms"], d["temperature"], stream=s)
            s.synchronize()
            got[t] = o
        except Exception as e:  # reported below, in the test's own thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(t,)) for t in range(len(devs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for ref, o in zip(refs, got):
        for k in ref:
            assert torch.equal(torch.nan_to_num(ref[k]), torch.nan_to_num(o[k])), k


def test_optional_outputs_omitted():
    # out_p, out_q and out_status are optional: without them the tokens and counts are the same
    # (every kernel that writes them checks for NULL), including fallback sequences.
    b = I.chain_gaussian(19, 6, 5, 4100, "bf16", 2.0, 1.0, 0.8)
    b.temperature[2] = -1.0
    d = BD.chain_to_device(b)
    args = (d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["temperature"])
    full = BD.sv_verify_chain(*args)
    bare = BD.sv_verify_chain(*args, want_pq=False, want_status=False)
    torch.cuda.synchronize()
    assert bare["p"] is None and bare["q"] is None and bare["status"] is None
    for k in ("tokens", "num_accepted"):
        assert torch.equal(full[k], bare[k]), k
