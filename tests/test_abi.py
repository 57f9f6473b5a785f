"""The C-ABI library: it loads, exports every symbol the header declares, and its host-side
validation rejects bad arguments before anything is launched (no GPU needed)."""

import ctypes
import os
import re

import pytest

from rejection_sampling_verify_chain_amd import binding as BD

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "specverify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(BD.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = BD.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert BD.version().startswith("specverify") and "gfx950" in BD.version()
    for st in (BD.SV_OK, BD.SV_ERR_NULL, BD.SV_ERR_SHAPE, BD.SV_ERR_DTYPE, BD.SV_ERR_WORKSPACE,
               BD.SV_ERR_LAUNCH, BD.SV_ERR_SCRATCH):
        assert BD.status_string(st).startswith("SV_")
    assert BD.status_string(99) == "unknown sv_status"


def test_workspace_sizes():
    lib = BD.load()
    f = lib.sv_verify_chain_workspace_bytes
    n = f(256, 7, 152064, BD.SV_F32)
    # per-chunk partials dominate: 3840 rows x 75 chunks x 16 bytes
    assert n >= 3840 * 75 * 16 and n % 256 == 0
    assert f(0, 4, 1000, BD.SV_F32) == 0 and f(1, 0, 1000, BD.SV_F32) == 0
    assert f(1, 65, 1000, BD.SV_F32) == 0 and f(1, 4, 0, BD.SV_F32) == 0
    assert f(1, 4, 1000, 7) == 0
    g = lib.sv_verify_tree_workspace_bytes
    assert g(16, 64, 32000, BD.SV_BF16) >= 16 * 64 * 16 * 16
    assert g(16, 4097, 32000, BD.SV_BF16) == 0
    a = lib.sv_chain_acceptance_rates_workspace_bytes
    assert a(256, 7, 152064, BD.SV_F32) >= 256 * 14 * 75 * 16
    assert a(1, 65, 1000, BD.SV_F32) == 0 and a(1, 4, 1000, 9) == 0
    sm = lib.sv_sample_workspace_bytes
    assert sm(256, 152064, BD.SV_F32) >= 256 * 75 * 16
    assert sm(0, 1000, BD.SV_F32) == 0 and sm(4, 0, BD.SV_BF16) == 0
    h = lib.sv_verify_chain_greedy_workspace_bytes
    assert h(256, 7, 152064, BD.SV_F32) >= 256 * 8 * 75 * 16
    assert h(1, 65, 1000, BD.SV_F32) == 0 and h(0, 4, 1000, BD.SV_BF16) == 0
    r = lib.sv_verify_chain_with_rates_workspace_bytes
    # the chain workspace plus one fp64 overlap sum per (sequence, position, chunk)
    assert r(256, 7, 152064, BD.SV_F32) >= f(256, 7, 152064, BD.SV_F32) + 256 * 7 * 75 * 8
    assert r(1, 65, 1000, BD.SV_F32) == 0 and r(1, 4, 1000, 7) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


CHAIN_ENTRIES = ["sv_verify_chain", "sv_verify_chain_lazy"]  # same signature and rules


def chain_call(entry="sv_verify_chain", **kw):
    a = dict(target=FAKE, draft=FAKE, dtype=BD.SV_F32, toks=FAKE, uni=FAKE, temp=FAKE, B=1,
             gamma=4, V=1000, out_tokens=FAKE, out_nacc=FAKE, out_p=None, out_q=None,
             out_status=None, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return getattr(BD.load(), entry)(*a.values())


def tree_call(**kw):
    a = dict(logits=FAKE, dtype=BD.SV_BF16, parents=FAKE, tokens=FAKE, n_trees=1, n_nodes=8,
             V=100, out_path=FAKE, out_tokens=FAKE, out_nacc=FAKE, out_g=None, out_status=None,
             ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return BD.load().sv_verify_tree(*a.values())


@pytest.mark.parametrize("entry", CHAIN_ENTRIES)
@pytest.mark.parametrize("field", ["target", "draft", "toks", "uni", "temp", "out_tokens",
                                   "out_nacc"])
def test_chain_null_pointers(field, entry):
    assert chain_call(entry, **{field: None}) == BD.SV_ERR_NULL


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), BD.SV_ERR_DTYPE),
    (dict(B=0), BD.SV_ERR_SHAPE), (dict(B=1 << 25), BD.SV_ERR_SHAPE),
    (dict(gamma=0), BD.SV_ERR_SHAPE), (dict(gamma=65), BD.SV_ERR_SHAPE),
    (dict(V=0), BD.SV_ERR_SHAPE), (dict(V=1 << 31), BD.SV_ERR_SHAPE),
    (dict(ws=None), BD.SV_ERR_WORKSPACE), (dict(ws_bytes=16), BD.SV_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x1010)), BD.SV_ERR_WORKSPACE),
])
@pytest.mark.parametrize("entry", CHAIN_ENTRIES)
def test_chain_validation(kw, status, entry):
    assert chain_call(entry, **kw) == status


def noalloc_call(**kw):
    a = dict(target=FAKE, draft=FAKE, dtype=BD.SV_F32, toks=FAKE, uni=FAKE, temp=FAKE, B=1,
             gamma=4, V=1000, out_tokens=FAKE, out_nacc=FAKE, out_p=None, out_q=None,
             out_status=None, stream=None)
    a.update(kw)
    return BD.load().sv_verify_chain_noalloc(*a.values())


@pytest.mark.parametrize("field", ["target", "draft", "toks", "uni", "temp", "out_tokens",
                                   "out_nacc"])
def test_noalloc_null_pointers(field):
    assert noalloc_call(**{field: None}) == BD.SV_ERR_NULL


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), BD.SV_ERR_DTYPE),
    (dict(B=0), BD.SV_ERR_SHAPE), (dict(gamma=65), BD.SV_ERR_SHAPE), (dict(V=0), BD.SV_ERR_SHAPE),
    # workspaces beyond the static scratch are refused before anything touches the GPU
    (dict(B=4096, gamma=7, V=152064), BD.SV_ERR_SCRATCH),
    (dict(B=1 << 21, gamma=1, V=1), BD.SV_ERR_SCRATCH),
])
def test_noalloc_validation(kw, status):
    assert noalloc_call(**kw) == status


def test_noalloc_scratch_limit_matches_workspace_sizes():
    f = BD.load().sv_verify_chain_workspace_bytes
    # the largest chain workload fits; sixteen times its batch does not
    assert f(256, 7, 152064, BD.SV_F32) <= BD.NOALLOC_SCRATCH_BYTES
    assert f(4096, 7, 152064, BD.SV_F32) > BD.NOALLOC_SCRATCH_BYTES


def rates_call(**kw):
    a = dict(target=FAKE, draft=FAKE, dtype=BD.SV_F32, toks=FAKE, uni=FAKE, temp=FAKE, B=1,
             gamma=4, V=1000, out_tokens=FAKE, out_nacc=FAKE, out_p=None, out_q=None,
             out_status=None, out_alpha=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return BD.load().sv_verify_chain_with_rates(*a.values())


@pytest.mark.parametrize("field", ["target", "draft", "toks", "uni", "temp", "out_tokens",
                                   "out_nacc", "out_alpha"])
def test_chain_with_rates_null_pointers(field):
    assert rates_call(**{field: None}) == BD.SV_ERR_NULL


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), BD.SV_ERR_DTYPE), (dict(gamma=65), BD.SV_ERR_SHAPE),
    (dict(V=0), BD.SV_ERR_SHAPE), (dict(ws=None), BD.SV_ERR_WORKSPACE),
    (dict(ws_bytes=16), BD.SV_ERR_WORKSPACE),
])
def test_chain_with_rates_validation(kw, status):
    assert rates_call(**kw) == status


def test_early_exit_has_no_rates():
    # The binding refuses the combination before it looks at any tensor.
    with pytest.raises(ValueError):
        BD.sv_verify_chain(None, None, None, None, None, lazy=True, want_rates=True)


def test_chain_with_rates_needs_its_own_workspace_size():
    lib = BD.load()
    plain = lib.sv_verify_chain_workspace_bytes(4, 5, 9000, BD.SV_BF16)
    assert lib.sv_verify_chain_with_rates_workspace_bytes(4, 5, 9000, BD.SV_BF16) > plain
    assert rates_call(B=4, gamma=5, V=9000, dtype=BD.SV_BF16, ws_bytes=plain) == BD.SV_ERR_WORKSPACE


@pytest.mark.parametrize("field", ["logits", "parents", "tokens", "out_path", "out_tokens",
                                   "out_nacc"])
def test_tree_null_pointers(field):
    assert tree_call(**{field: None}) == BD.SV_ERR_NULL


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=-1), BD.SV_ERR_DTYPE),
    (dict(n_trees=0), BD.SV_ERR_SHAPE), (dict(n_nodes=0), BD.SV_ERR_SHAPE),
    (dict(n_nodes=4097), BD.SV_ERR_SHAPE), (dict(V=0), BD.SV_ERR_SHAPE),
    (dict(ws=None), BD.SV_ERR_WORKSPACE), (dict(ws_bytes=0), BD.SV_ERR_WORKSPACE),
])
def test_tree_validation(kw, status):
    assert tree_call(**kw) == status


def greedy_call(**kw):
    a = dict(target=FAKE, dtype=BD.SV_BF16, toks=FAKE, B=2, gamma=4, V=1000, out_tokens=FAKE,
             out_nacc=FAKE, out_g=None, out_status=None, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return BD.load().sv_verify_chain_greedy(*a.values())


@pytest.mark.parametrize("field", ["target", "toks", "out_tokens", "out_nacc"])
def test_greedy_null_pointers(field):
    assert greedy_call(**{field: None}) == BD.SV_ERR_NULL


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), BD.SV_ERR_DTYPE),
    (dict(B=0), BD.SV_ERR_SHAPE), (dict(gamma=0), BD.SV_ERR_SHAPE), (dict(gamma=65), BD.SV_ERR_SHAPE),
    (dict(V=0), BD.SV_ERR_SHAPE), (dict(ws=None), BD.SV_ERR_WORKSPACE),
    (dict(ws_bytes=16), BD.SV_ERR_WORKSPACE), (dict(ws=ctypes.c_void_p(0x1010)), BD.SV_ERR_WORKSPACE),
])
def test_greedy_host_validation(kw, status):
    assert greedy_call(**kw) == status


def alpha_call(**kw):
    a = dict(target=FAKE, draft=FAKE, dtype=BD.SV_F32, temp=FAKE, B=2, gamma=4, V=1000,
             out_alpha=FAKE, out_status=None, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return BD.load().sv_chain_acceptance_rates(*a.values())


@pytest.mark.parametrize("field", ["target", "draft", "temp", "out_alpha"])
def test_alpha_null_pointers(field):
    assert alpha_call(**{field: None}) == BD.SV_ERR_NULL


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), BD.SV_ERR_DTYPE), (dict(B=0), BD.SV_ERR_SHAPE), (dict(gamma=65), BD.SV_ERR_SHAPE),
    (dict(V=-1), BD.SV_ERR_SHAPE), (dict(ws_bytes=0), BD.SV_ERR_WORKSPACE),
])
def test_alpha_host_validation(kw, status):
    assert alpha_call(**kw) == status


def sample_call(**kw):
    a = dict(logits=FAKE, dtype=BD.SV_BF16, temp=FAKE, uni=FAKE, rows=3, V=1000, out_tokens=FAKE,
             out_prob=None, out_status=None, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return BD.load().sv_sample(*a.values())


@pytest.mark.parametrize("field", ["logits", "temp", "uni", "out_tokens"])
def test_sample_null_pointers(field):
    assert sample_call(**{field: None}) == BD.SV_ERR_NULL


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=4), BD.SV_ERR_DTYPE), (dict(rows=0), BD.SV_ERR_SHAPE), (dict(V=0), BD.SV_ERR_SHAPE),
    (dict(ws=None), BD.SV_ERR_WORKSPACE), (dict(ws_bytes=8), BD.SV_ERR_WORKSPACE),
])
def test_sample_host_validation(kw, status):
    assert sample_call(**kw) == status


def kv_call(**kw):
    a = dict(src=ctypes.c_void_p(0x100000), dst=ctypes.c_void_p(0x900000), row_bytes=1024, n=2,
             src_rows=8, dst_rows=16, path=None, path_len=0, k=FAKE, start=FAKE, status=None,
             stream=None)
    a.update(kw)
    return BD.load().sv_compact_accepted(*a.values())


@pytest.mark.parametrize("field", ["src", "dst", "k", "start"])
def test_kv_null_pointers(field):
    assert kv_call(**{field: None}) == BD.SV_ERR_NULL


@pytest.mark.parametrize("kw", [dict(n=0), dict(row_bytes=0), dict(src_rows=0), dict(dst_rows=0),
                                dict(path=FAKE, path_len=0),
                                dict(dst=ctypes.c_void_p(0x100000 + 4096))])  # overlaps src
def test_kv_host_validation(kw):
    assert kv_call(**kw) == BD.SV_ERR_SHAPE


def test_read_probe_sizes_and_validation():
    lib = BD.load()
    group = 128 * 1024  # bytes one probe workgroup reads
    assert lib.sv_read_probe_out_words(16) == 1
    assert lib.sv_read_probe_out_words(group) == 1
    assert lib.sv_read_probe_out_words(group + 16) == 2
    assert lib.sv_read_probe_out_words(0) == 0 and lib.sv_read_probe_out_words(24) == 0
    assert lib.sv_read_probe_out_words(-16) == 0
    # Every call below fails validation before any launch.
    assert lib.sv_read_probe(None, 16, FAKE, None) == BD.SV_ERR_NULL
    assert lib.sv_read_probe(FAKE, 16, None, None) == BD.SV_ERR_NULL
    assert lib.sv_read_probe(FAKE, 24, FAKE, None) == BD.SV_ERR_SHAPE
    assert lib.sv_read_probe(ctypes.c_void_p(0x1008), 16, FAKE, None) == BD.SV_ERR_SHAPE
