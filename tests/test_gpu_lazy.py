"""GPU parity of sv_verify_chain_lazy (early exit) against the oracle and against sv_verify_chain.

The early-exit entry point takes the positions in order and reads no row after the cut.  For
inputs whose rows are all finite its tokens, k and status must be sv_verify_chain's bit for bit
and its p, q at positions i <= k too; after the cut p and q are NaN where the row was not read.
Most tests force each of the two early-exit forms (SPECVERIFY_CHAIN_PATH=lazy: one workgroup per
sequence; staged: one launch per position), whatever the batch; the threshold and full-size tests
leave the choice to the library.
"""

import numpy as np
import pytest
import torch

from parity import BAND_LIMITS, assert_band_limit, check_chain
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["lazy", "staged"])
def forced(request, monkeypatch):
    """Both early-exit forms: one workgroup per sequence taking the positions in order, and one
    launch per position across the chip."""
    monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", request.param)
    return request.param


def run(batch, lazy=True, d=None):
    d = BD.chain_to_device(batch) if d is None else d
    out = BD.sv_verify_chain(d["target"], d["draft"], d["draft_tokens"], d["uniforms"],
                             d["temperature"], lazy=lazy)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def report(name, counts):
    print(f"[parity] lazy {name}: {counts}", flush=True)


def assert_same_as_eager(lazy, eager):
    """Bit-equal tokens, k and status; p and q bit-equal at i <= k, NaN or equal after."""
    for key in ("tokens", "num_accepted", "status"):
        assert np.array_equal(lazy[key], eager[key]), key
    k = eager["num_accepted"]
    pos = np.arange(lazy["p"].shape[1])[None, :]
    upto = pos <= k[:, None]
    for key in ("p", "q"):
        a, b = lazy[key], eager[key]
        assert np.array_equal(a[upto], b[upto], equal_nan=True), key
        after = ~upto
        assert np.all(np.isnan(a[after]) | (a[after] == b[after])), key


def check_both(batch, name, seqs=None, refs=None):
    """Early exit against the oracle and against the eager entry point on the same buffers."""
    d = BD.chain_to_device(batch)
    lazy = run(batch, True, d)
    counts = check_chain(batch, lazy, seqs, lazy=True, refs=refs)
    report(name, counts)
    if seqs is None and batch.name in BAND_LIMITS:
        assert_band_limit(batch.name, counts)
    assert_same_as_eager(lazy, run(batch, False, d))
    return lazy


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 63, 1000, 2047, 2048, 2049, 5003, 8191])
def test_edge_shapes(forced, dtype, V):
    for B, gamma, T in ((1, 1, 1.0), (3, 2, 0.5), (17, 7, 2.0)):
        b = I.chain_gaussian(V * 37 + B, B, gamma, V, dtype, 2.0, 1.0, T)
        check_both(b, f"gauss {dtype} V={V} B={B} g={gamma}")


def test_cuts_at_every_position(forced):
    # Weak drafts cut early, strong ones late: across 64 sequences every k in 0..gamma occurs,
    # so the kernel leaves its loop at each position and also runs to the bonus draw.
    b = I.chain_gaussian(71, 64, 5, 3000, "f32", 2.0, 0.6, 1.0, draft_scale=0.95)
    out = check_both(b, "every cut")
    assert set(out["num_accepted"].tolist()) == set(range(6))


def test_gamma_max_and_all_accept(forced):
    rng = np.random.default_rng(0)
    t = rng.normal(scale=2.0, size=(2, 65, 300)).astype(np.float32)
    b = I.chain_from_logits(6, t, t[:, :64], 0.9)
    out = check_both(b, "gamma=64 p==q")
    assert np.all(out["num_accepted"] == 64)


def test_masked_logits_and_disjoint_support(forced):
    rng = np.random.default_rng(1)
    B, g, V = 6, 3, 3000
    t = rng.normal(scale=2.0, size=(B, g + 1, V)).astype(np.float32)
    d = (t[:, :g] + rng.normal(size=(B, g, V))).astype(np.float32)
    t[rng.random(t.shape) < 0.3] = -np.inf
    d[rng.random(d.shape) < 0.3] = -np.inf
    d[0, 0, :1500] = -np.inf
    t[0, 0, 1500:] = -np.inf
    out = check_both(I.chain_from_logits(7, t, d, 1.0), "masked")
    assert out["num_accepted"][0] == 0 and out["tokens"][0, 0] < 1500


@pytest.mark.parametrize("T", [1e-30, 1e-3, 50.0, 1e30])
def test_extreme_temperatures(forced, T):
    check_both(I.chain_gaussian(9, 5, 4, 777, "f32", 2.0, 1.0, T), f"T={T}")


def test_zipf_b64_g4_v128256_full(forced):
    b = I.chain_zipf_b64_v128256()
    check_both(b, b.name)


def test_host_checked_data_errors(forced):
    # Errors found without reading a logit row give sv_verify_chain's fallback and status.
    b = I.chain_gaussian(8, 4, 3, 500, "f32", 2.0, 1.0, 1.0)
    b.draft_tokens[0, 2] = 500
    b.temperature[1] = 0.0
    b.uniforms[2, 3] = 1.0
    out = check_both(b, "host-checked errors")
    assert list(out["status"]) == [BD.ROW_TOKEN_RANGE, BD.ROW_BAD_TEMPERATURE,
                                   BD.ROW_BAD_UNIFORM, 0]


def _poison(batch, seq, first_pos):
    """NaN in every row of sequence seq from position first_pos on (target rows up to gamma)."""
    batch.target[seq, first_pos:, 5] = np.nan
    batch.draft[seq, first_pos:, 7] = np.nan


def test_nonfinite_rows_before_the_cut_fall_back(forced):
    b = I.chain_gaussian(12, 8, 4, 2500, "f32", 2.0, 1.0, 1.0)
    clean = run(b)
    for s in range(8):  # the NaN sits at or before the cut: the row is read
        b.target[s, min(int(clean["num_accepted"][s]), s % 4), 11] = np.nan
    out = run(b)
    assert np.all(out["status"] == BD.ROW_NONFINITE)
    report("non-finite before the cut", check_chain(b, out, lazy=True))


def test_nonfinite_rows_after_the_cut_are_not_read(forced):
    b = I.chain_gaussian(13, 32, 6, 3000, "f32", 2.0, 1.0, 0.9)
    clean = run(b)
    k = clean["num_accepted"]
    cut = np.flatnonzero(k < 6)
    assert len(cut) >= 8
    for s in cut:
        _poison(b, s, int(k[s]) + 1)
    poisoned = run(b)
    for key in clean:
        assert np.array_equal(poisoned[key], clean[key], equal_nan=True), key
    # sv_verify_chain reads every row and falls back on the same input, as the oracle does.
    eager = run(b, lazy=False)
    assert np.all(eager["status"][cut] == BD.ROW_NONFINITE)
    check_chain(b, eager)


def test_small_batch_runs_as_verify_chain():
    # Below 128 sequences (no forcing) the entry point is sv_verify_chain: every p, q evaluated.
    b = I.chain_gaussian(14, 127, 4, 4096, "bf16", 2.0, 1.0, 1.0)
    d = BD.chain_to_device(b)
    lazy, eager = run(b, True, d), run(b, False, d)
    for key in lazy:
        assert np.array_equal(lazy[key], eager[key], equal_nan=True), key
    assert not np.any(np.isnan(lazy["p"]))


def test_batch_threshold_takes_early_exit():
    # From 256 sequences on, narrow rows take the one-workgroup form: p, q NaN after the cut.
    b = I.chain_gaussian(15, 256, 4, 4096, "bf16", 2.0, 1.0, 1.0)
    out = check_both(b, "B=256 auto")
    k = out["num_accepted"]
    after = np.arange(4)[None, :] > k[:, None]
    assert after.any() and np.all(np.isnan(out["p"][after])) and np.all(np.isnan(out["q"][after]))


@pytest.mark.parametrize("form", ["auto", "staged", "lazy"])
def test_gauss_b256_g7_v152064_full(gauss_b256, form, monkeypatch):
    # Full workload, every sequence: the library's own choice at this batch (the staged form),
    # and each early-exit form forced.
    if form != "auto":
        monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", form)
    b, refs = gauss_b256
    out = check_both(b, f"{b.name} {form}", refs=refs)
    after = np.arange(7)[None, :] > out["num_accepted"][:, None]
    assert np.all(np.isnan(out["p"][after]))


def test_deterministic(forced):
    b = I.chain_gaussian(16, 9, 5, 6000, "bf16", 2.0, 1.0, 0.7)
    d = BD.chain_to_device(b)
    first = run(b, True, d)
    for _ in range(3):
        again = run(b, True, d)
        for key in first:
            assert np.array_equal(first[key], again[key], equal_nan=True), key



@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_rows_run_as_verify_chain(forced, dtype):
    # Rows that are not 16-byte aligned have no early-exit form: the entry point runs
    # sv_verify_chain (every p and q evaluated), forced or not.
    b = I.chain_gaussian(18, 4, 3, 4096, dtype, 2.0, 1.0, 1.0)
    d = BD.chain_to_device(b)

    def shifted(t):
        flat = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = flat[1:].view(t.shape)
        v.copy_(t)
        return v

    tgt, drf = shifted(d["target"]), shifted(d["draft"])
    out = BD.sv_verify_chain(tgt, drf, d["draft_tokens"], d["uniforms"], d["temperature"],
                             lazy=True)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in out.items()}
    assert not np.isnan(out["p"]).any()
    report(f"unaligned {dtype}", check_chain(b, out))


def test_optional_outputs_omitted(forced):
    b = I.chain_gaussian(20, 6, 5, 4100, "bf16", 2.0, 1.0, 0.8)
    b.temperature[2] = -1.0
    d = BD.chain_to_device(b)
    args = (d["target"], d["draft"], d["draft_tokens"], d["uniforms"], d["temperature"])
    full = BD.sv_verify_chain(*args, lazy=True)
    bare = BD.sv_verify_chain(*args, lazy=True, want_pq=False, want_status=False)
    torch.cuda.synchronize()
    for k in ("tokens", "num_accepted"):
        assert torch.equal(full[k], bare[k]), k


def test_large_batch_small_rows(monkeypatch):
    # 4096 sequences of short rows: large grids on every path (eager, and both early-exit forms).
    b = I.chain_gaussian(28, 4096, 3, 100, "f32", 2.0, 1.0, 1.0)
    d = BD.chain_to_device(b)
    eager = run(b, False, d)
    check_chain(b, eager, list(range(0, 4096, 37)) + [4095])
    for form in ("lazy", "staged"):
        monkeypatch.setenv("SPECVERIFY_CHAIN_PATH", form)
        assert_same_as_eager(run(b, True, d), eager)
