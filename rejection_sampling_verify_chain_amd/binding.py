"""ctypes binding of libspecverify: argument marshalling only.

Each function takes torch tensors that already live on the GPU, checks that
their dtypes, shapes and contiguity match the C ABI declared in
include/specverify.h, allocates any output or workspace tensor the caller did
not pass, and calls the entry point of the same name on the current torch
stream.  Every step of the verify path runs in the library's HIP kernels; if
the library is missing this module raises instead of computing anything
itself.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecverify.so")

SV_F32, SV_BF16 = 0, 1
SV_OK, SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_DTYPE, SV_ERR_WORKSPACE, SV_ERR_LAUNCH = 0, 1, 2, 3, 5, 6
SV_ERR_SCRATCH = 7
NOALLOC_SCRATCH_BYTES = 32 << 20  # SV_NOALLOC_SCRATCH_BYTES
ROW_TOKEN_RANGE, ROW_NONFINITE, ROW_RESIDUAL_ZERO = 1, 2, 4
ROW_BAD_TREE, ROW_BAD_TEMPERATURE, ROW_BAD_UNIFORM = 8, 16, 32
ROW_BAD_INDEX = 64

EXPORTS = (
    "sv_version", "sv_status_string",
    "sv_verify_chain_workspace_bytes", "sv_verify_chain",
    "sv_verify_chain_with_rates_workspace_bytes", "sv_verify_chain_with_rates",
    "sv_verify_chain_lazy", "sv_verify_chain_noalloc",
    "sv_verify_tree_workspace_bytes", "sv_verify_tree",
    "sv_verify_chain_greedy_workspace_bytes", "sv_verify_chain_greedy",
    "sv_chain_acceptance_rates_workspace_bytes", "sv_chain_acceptance_rates",
    "sv_sample_workspace_bytes", "sv_sample",
    "sv_compact_accepted",
    "sv_trace_start", "sv_trace_stop", "sv_trace_kernels", "sv_trace_get",
    "sv_read_probe_out_words", "sv_read_probe",
)

_DTYPE = {torch.float32: SV_F32, torch.bfloat16: SV_BF16}
_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def load():
    """Load libspecverify.so (after torch, so the HIP runtime torch loaded is the one used)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m rejection_sampling_verify_chain_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.sv_version.restype = ctypes.c_char_p
    lib.sv_version.argtypes = []
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_status_string.argtypes = [ctypes.c_int]
    lib.sv_verify_chain_workspace_bytes.restype = sz
    lib.sv_verify_chain_workspace_bytes.argtypes = [i32, i32, i64, ctypes.c_int]
    lib.sv_verify_chain.restype = ctypes.c_int
    lib.sv_verify_chain.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, i32, i32, i64,
                                    vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sv_verify_chain_lazy.restype = ctypes.c_int
    lib.sv_verify_chain_lazy.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, i32, i32, i64,
                                         vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sv_verify_chain_noalloc.restype = ctypes.c_int
    lib.sv_verify_chain_noalloc.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, i32, i32, i64,
                                            vp, vp, vp, vp, vp, vp]
    lib.sv_verify_chain_with_rates_workspace_bytes.restype = sz
    lib.sv_verify_chain_with_rates_workspace_bytes.argtypes = [i32, i32, i64, ctypes.c_int]
    lib.sv_verify_chain_with_rates.restype = ctypes.c_int
    lib.sv_verify_chain_with_rates.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, i32, i32, i64,
                                               vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sv_verify_tree_workspace_bytes.restype = sz
    lib.sv_verify_tree_workspace_bytes.argtypes = [i32, i32, i64, ctypes.c_int]
    lib.sv_verify_tree.restype = ctypes.c_int
    lib.sv_verify_tree.argtypes = [vp, ctypes.c_int, vp, vp, i32, i32, i64,
                                   vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sv_verify_chain_greedy_workspace_bytes.restype = sz
    lib.sv_verify_chain_greedy_workspace_bytes.argtypes = [i32, i32, i64, ctypes.c_int]
    lib.sv_verify_chain_greedy.restype = ctypes.c_int
    lib.sv_verify_chain_greedy.argtypes = [vp, ctypes.c_int, vp, i32, i32, i64,
                                           vp, vp, vp, vp, vp, sz, vp]
    lib.sv_chain_acceptance_rates_workspace_bytes.restype = sz
    lib.sv_chain_acceptance_rates_workspace_bytes.argtypes = [i32, i32, i64, ctypes.c_int]
    lib.sv_chain_acceptance_rates.restype = ctypes.c_int
    lib.sv_chain_acceptance_rates.argtypes = [vp, vp, ctypes.c_int, vp, i32, i32, i64,
                                              vp, vp, vp, sz, vp]
    lib.sv_sample_workspace_bytes.restype = sz
    lib.sv_sample_workspace_bytes.argtypes = [i32, i64, ctypes.c_int]
    lib.sv_sample.restype = ctypes.c_int
    lib.sv_sample.argtypes = [vp, ctypes.c_int, vp, vp, i32, i64, vp, vp, vp, vp, sz, vp]
    lib.sv_compact_accepted.restype = ctypes.c_int
    lib.sv_compact_accepted.argtypes = [vp, vp, i64, i32, i32, i32, vp, i32, vp, vp, vp, vp]
    lib.sv_trace_start.restype = ctypes.c_int
    lib.sv_trace_start.argtypes = [ctypes.c_int]
    lib.sv_trace_stop.restype = ctypes.c_int
    lib.sv_trace_stop.argtypes = []
    lib.sv_trace_kernels.restype = ctypes.c_int
    lib.sv_trace_kernels.argtypes = []
    lib.sv_trace_get.restype = ctypes.c_int
    lib.sv_trace_get.argtypes = [ctypes.c_int, ctypes.c_char_p, sz, ctypes.POINTER(ctypes.c_int),
                                 ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_double)]
    lib.sv_read_probe_out_words.restype = sz
    lib.sv_read_probe_out_words.argtypes = [ctypes.c_int64]
    lib.sv_read_probe.restype = ctypes.c_int
    lib.sv_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_void_p]
    _lib = lib
    return lib


def trace_start(capacity):
    if load().sv_trace_start(int(capacity)) != 0:
        raise RuntimeError("sv_trace_start failed")


def trace_stop():
    return int(load().sv_trace_stop())


def trace_kernels():
    """{kernel name: {"launches", "total_ms", "min_ms", "max_ms", "avg_ms"}} of the last trace."""
    lib = load()
    n = lib.sv_trace_kernels()
    if n < 0:
        raise RuntimeError("sv_trace_kernels failed")
    out = {}
    for i in range(n):
        name = ctypes.create_string_buffer(64)
        la, tot, mn, mx = ctypes.c_int(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        lib.sv_trace_get(i, name, 64, ctypes.byref(la), ctypes.byref(tot), ctypes.byref(mn),
                         ctypes.byref(mx))
        out[name.value.decode()] = {"launches": la.value, "total_ms": tot.value,
                                    "min_ms": mn.value, "max_ms": mx.value,
                                    "avg_ms": tot.value / max(1, la.value)}
    return out


def version():
    return load().sv_version().decode()


def status_string(status):
    return load().sv_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, name, dtype, shape, device):
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out(t, name, dtype, shape, device):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _check(t, name, dtype, shape, device)
    return t


def chain_workspace_bytes(B, gamma, V, dtype):
    return int(load().sv_verify_chain_workspace_bytes(B, gamma, V, _DTYPE[dtype]))


def chain_with_rates_workspace_bytes(B, gamma, V, dtype):
    return int(load().sv_verify_chain_with_rates_workspace_bytes(B, gamma, V, _DTYPE[dtype]))


def tree_workspace_bytes(n_trees, n_nodes, V, dtype):
    return int(load().sv_verify_tree_workspace_bytes(n_trees, n_nodes, V, _DTYPE[dtype]))


def chain_greedy_workspace_bytes(B, gamma, V, dtype):
    return int(load().sv_verify_chain_greedy_workspace_bytes(B, gamma, V, _DTYPE[dtype]))


def acceptance_rates_workspace_bytes(B, gamma, V, dtype):
    return int(load().sv_chain_acceptance_rates_workspace_bytes(B, gamma, V, _DTYPE[dtype]))


def sample_workspace_bytes(rows, V, dtype):
    return int(load().sv_sample_workspace_bytes(rows, V, _DTYPE[dtype]))


def workspace(nbytes, device):
    """A device byte buffer for the library's scratch (torch allocations are 256-byte aligned)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def sv_verify_chain(target, draft, draft_tokens, uniforms, temperature, *, out_tokens=None,
                    out_num_accepted=None, out_p=None, out_q=None, out_status=None,
                    workspace_buf=None, stream=None, want_pq=True, want_status=True,
                    want_rates=False, out_alpha=None, lazy=False):
    """Chain verification through the C ABI.

    target [B, gamma+1, V] and draft [B, gamma, V] (fp32 or bf16), draft_tokens int32
    [B, gamma], uniforms fp32 [B, gamma+1], temperature fp32 [B].  Returns a dict of the
    output tensors (tokens, num_accepted, p, q, status); the call is asynchronous.  With
    want_rates (or an out_alpha tensor) it calls sv_verify_chain_with_rates and the dict also
    holds alpha fp32 [B, gamma]; with lazy it calls sv_verify_chain_lazy (early exit).
    """
    lib = load()
    rates = want_rates or out_alpha is not None
    if rates and lazy:
        raise ValueError("the early-exit entry point has no acceptance rates")
    if target.dtype not in _DTYPE:
        raise ValueError(f"logits must be float32 or bfloat16, got {target.dtype}")
    dev = target.device
    B, g1, V = target.shape
    gamma = g1 - 1
    _check(target, "target", None, (B, gamma + 1, V), dev)
    _check(draft, "draft", target.dtype, (B, gamma, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, gamma), dev)
    _check(uniforms, "uniforms", torch.float32, (B, gamma + 1), dev)
    _check(temperature, "temperature", torch.float32, (B,), dev)
    out_tokens = _out(out_tokens, "out_tokens", torch.int32, (B, gamma + 1), dev)
    out_num_accepted = _out(out_num_accepted, "out_num_accepted", torch.int32, (B,), dev)
    if want_pq or out_p is not None:
        out_p = _out(out_p, "out_p", torch.float32, (B, gamma), dev)
    if want_pq or out_q is not None:
        out_q = _out(out_q, "out_q", torch.float32, (B, gamma), dev)
    if want_status or out_status is not None:
        out_status = _out(out_status, "out_status", torch.int32, (B,), dev)
    if rates:
        out_alpha = _out(out_alpha, "out_alpha", torch.float32, (B, gamma), dev)
        need = chain_with_rates_workspace_bytes(B, gamma, V, target.dtype)
    else:
        need = chain_workspace_bytes(B, gamma, V, target.dtype)
    if workspace_buf is None:
        workspace_buf = workspace(need, dev)
    args = [_ptr(target), _ptr(draft), _DTYPE[target.dtype], _ptr(draft_tokens), _ptr(uniforms),
            _ptr(temperature), B, gamma, V, _ptr(out_tokens), _ptr(out_num_accepted), _ptr(out_p),
            _ptr(out_q), _ptr(out_status)]
    if rates:
        name = "sv_verify_chain_with_rates"
        st = lib.sv_verify_chain_with_rates(*args, _ptr(out_alpha), _ptr(workspace_buf),
                                            workspace_buf.numel(), _stream(stream))
    else:
        name = "sv_verify_chain_lazy" if lazy else "sv_verify_chain"
        st = getattr(lib, name)(*args, _ptr(workspace_buf), workspace_buf.numel(),
                                _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, name)
    out = {"tokens": out_tokens, "num_accepted": out_num_accepted, "p": out_p, "q": out_q,
           "status": out_status}
    if rates:
        out["alpha"] = out_alpha
    return out


def sv_verify_chain_noalloc(target, draft, draft_tokens, uniforms, temperature, *, out_tokens,
                            out_num_accepted, out_p=None, out_q=None, out_status=None,
                            stream=None):
    """Chain verification through the entry point that allocates nothing.

    Same inputs as sv_verify_chain; every output is the caller's (out_p, out_q and out_status
    may be None, passed as NULL), this function creates no tensor, and the library takes its
    workspace from its static device scratch.  Raises SpecVerifyError with SV_ERR_SCRATCH when
    the shape's workspace exceeds NOALLOC_SCRATCH_BYTES.  Returns the dict of output tensors.
    """
    lib = load()
    if target.dtype not in _DTYPE:
        raise ValueError(f"logits must be float32 or bfloat16, got {target.dtype}")
    dev = target.device
    B, g1, V = target.shape
    gamma = g1 - 1
    _check(target, "target", None, (B, gamma + 1, V), dev)
    _check(draft, "draft", target.dtype, (B, gamma, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, gamma), dev)
    _check(uniforms, "uniforms", torch.float32, (B, gamma + 1), dev)
    _check(temperature, "temperature", torch.float32, (B,), dev)
    _check(out_tokens, "out_tokens", torch.int32, (B, gamma + 1), dev)
    _check(out_num_accepted, "out_num_accepted", torch.int32, (B,), dev)
    for t, name, dt, shape in ((out_p, "out_p", torch.float32, (B, gamma)),
                               (out_q, "out_q", torch.float32, (B, gamma)),
                               (out_status, "out_status", torch.int32, (B,))):
        if t is not None:
            _check(t, name, dt, shape, dev)
    st = lib.sv_verify_chain_noalloc(
        _ptr(target), _ptr(draft), _DTYPE[target.dtype], _ptr(draft_tokens), _ptr(uniforms),
        _ptr(temperature), B, gamma, V, _ptr(out_tokens), _ptr(out_num_accepted), _ptr(out_p),
        _ptr(out_q), _ptr(out_status), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_verify_chain_noalloc")
    return {"tokens": out_tokens, "num_accepted": out_num_accepted, "p": out_p, "q": out_q,
            "status": out_status}


def sv_verify_tree(logits, parents, node_tokens, *, out_path=None, out_tokens=None,
                   out_num_accepted=None, out_node_argmax=None, out_status=None,
                   workspace_buf=None, stream=None, want_argmax=True, want_status=True):
    """Greedy token-tree verification through the C ABI.

    logits [n_trees, n_nodes, V] (fp32 or bf16), parents and node_tokens int32
    [n_trees, n_nodes].  Returns a dict (path, tokens, num_accepted, node_argmax, status).
    """
    lib = load()
    if logits.dtype not in _DTYPE:
        raise ValueError(f"logits must be float32 or bfloat16, got {logits.dtype}")
    dev = logits.device
    n_trees, n_nodes, V = logits.shape
    _check(logits, "logits", None, (n_trees, n_nodes, V), dev)
    _check(parents, "parents", torch.int32, (n_trees, n_nodes), dev)
    _check(node_tokens, "node_tokens", torch.int32, (n_trees, n_nodes), dev)
    out_path = _out(out_path, "out_path", torch.int32, (n_trees, n_nodes), dev)
    out_tokens = _out(out_tokens, "out_tokens", torch.int32, (n_trees, n_nodes), dev)
    out_num_accepted = _out(out_num_accepted, "out_num_accepted", torch.int32, (n_trees,), dev)
    if want_argmax or out_node_argmax is not None:
        out_node_argmax = _out(out_node_argmax, "out_node_argmax", torch.int32,
                               (n_trees, n_nodes), dev)
    if want_status or out_status is not None:
        out_status = _out(out_status, "out_status", torch.int32, (n_trees,), dev)
    need = tree_workspace_bytes(n_trees, n_nodes, V, logits.dtype)
    if workspace_buf is None:
        workspace_buf = workspace(need, dev)
    st = lib.sv_verify_tree(
        _ptr(logits), _DTYPE[logits.dtype], _ptr(parents), _ptr(node_tokens), n_trees, n_nodes,
        V, _ptr(out_path), _ptr(out_tokens), _ptr(out_num_accepted), _ptr(out_node_argmax),
        _ptr(out_status), _ptr(workspace_buf), workspace_buf.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_verify_tree")
    return {"path": out_path, "tokens": out_tokens, "num_accepted": out_num_accepted,
            "node_argmax": out_node_argmax, "status": out_status}


def sv_verify_chain_greedy(target, draft_tokens, *, out_tokens=None, out_num_accepted=None,
                           out_argmax=None, out_status=None, workspace_buf=None, stream=None,
                           want_argmax=True, want_status=True):
    """Greedy chain verification through the C ABI.

    target [B, gamma+1, V] (fp32 or bf16), draft_tokens int32 [B, gamma].  Returns a dict
    (tokens, num_accepted, argmax, status); the call is asynchronous.
    """
    lib = load()
    if target.dtype not in _DTYPE:
        raise ValueError(f"logits must be float32 or bfloat16, got {target.dtype}")
    dev = target.device
    B, g1, V = target.shape
    gamma = g1 - 1
    _check(target, "target", None, (B, gamma + 1, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, gamma), dev)
    out_tokens = _out(out_tokens, "out_tokens", torch.int32, (B, gamma + 1), dev)
    out_num_accepted = _out(out_num_accepted, "out_num_accepted", torch.int32, (B,), dev)
    if want_argmax or out_argmax is not None:
        out_argmax = _out(out_argmax, "out_argmax", torch.int32, (B, gamma + 1), dev)
    if want_status or out_status is not None:
        out_status = _out(out_status, "out_status", torch.int32, (B,), dev)
    need = chain_greedy_workspace_bytes(B, gamma, V, target.dtype)
    if workspace_buf is None:
        workspace_buf = workspace(need, dev)
    st = lib.sv_verify_chain_greedy(
        _ptr(target), _DTYPE[target.dtype], _ptr(draft_tokens), B, gamma, V, _ptr(out_tokens),
        _ptr(out_num_accepted), _ptr(out_argmax), _ptr(out_status), _ptr(workspace_buf),
        workspace_buf.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_verify_chain_greedy")
    return {"tokens": out_tokens, "num_accepted": out_num_accepted, "argmax": out_argmax,
            "status": out_status}


def sv_chain_acceptance_rates(target, draft, temperature, *, out_alpha=None, out_status=None,
                              workspace_buf=None, stream=None, want_status=True):
    """Per-position acceptance rates through the C ABI.

    target [B, gamma+1, V] and draft [B, gamma, V] (fp32 or bf16), temperature fp32 [B].
    Returns a dict (alpha fp32 [B, gamma], status int32 [B, gamma]); the call is asynchronous.
    """
    lib = load()
    if target.dtype not in _DTYPE:
        raise ValueError(f"logits must be float32 or bfloat16, got {target.dtype}")
    dev = target.device
    B, g1, V = target.shape
    gamma = g1 - 1
    _check(target, "target", None, (B, gamma + 1, V), dev)
    _check(draft, "draft", target.dtype, (B, gamma, V), dev)
    _check(temperature, "temperature", torch.float32, (B,), dev)
    out_alpha = _out(out_alpha, "out_alpha", torch.float32, (B, gamma), dev)
    if want_status or out_status is not None:
        out_status = _out(out_status, "out_status", torch.int32, (B, gamma), dev)
    need = acceptance_rates_workspace_bytes(B, gamma, V, target.dtype)
    if workspace_buf is None:
        workspace_buf = workspace(need, dev)
    st = lib.sv_chain_acceptance_rates(
        _ptr(target), _ptr(draft), _DTYPE[target.dtype], _ptr(temperature), B, gamma, V,
        _ptr(out_alpha), _ptr(out_status), _ptr(workspace_buf), workspace_buf.numel(),
        _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_chain_acceptance_rates")
    return {"alpha": out_alpha, "status": out_status}


def sv_sample(logits, temperature, uniforms, *, out_tokens=None, out_prob=None, out_status=None,
              workspace_buf=None, stream=None, want_prob=True, want_status=True):
    """Draft-side sampler through the C ABI.

    logits [rows, V] (fp32 or bf16), temperature and uniforms fp32 [rows].  Returns a dict
    (tokens, prob, status); the call is asynchronous.
    """
    lib = load()
    if logits.dtype not in _DTYPE:
        raise ValueError(f"logits must be float32 or bfloat16, got {logits.dtype}")
    dev = logits.device
    rows, V = logits.shape
    _check(logits, "logits", None, (rows, V), dev)
    _check(temperature, "temperature", torch.float32, (rows,), dev)
    _check(uniforms, "uniforms", torch.float32, (rows,), dev)
    out_tokens = _out(out_tokens, "out_tokens", torch.int32, (rows,), dev)
    if want_prob or out_prob is not None:
        out_prob = _out(out_prob, "out_prob", torch.float32, (rows,), dev)
    if want_status or out_status is not None:
        out_status = _out(out_status, "out_status", torch.int32, (rows,), dev)
    need = sample_workspace_bytes(rows, V, logits.dtype)
    if workspace_buf is None:
        workspace_buf = workspace(need, dev)
    st = lib.sv_sample(_ptr(logits), _DTYPE[logits.dtype], _ptr(temperature), _ptr(uniforms), rows,
                       V, _ptr(out_tokens), _ptr(out_prob), _ptr(out_status),
                       _ptr(workspace_buf), workspace_buf.numel(), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_sample")
    return {"tokens": out_tokens, "prob": out_prob, "status": out_status}


def read_probe_out_words(nbytes):
    return int(load().sv_read_probe_out_words(int(nbytes)))


def sv_read_probe(buf, *, out=None, stream=None):
    """Plain streaming read of a contiguous device tensor (the read ceiling the verify kernels
    are set beside); returns the int32 tensor of per-workgroup XORs of the words read."""
    lib = load()
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    words = read_probe_out_words(nbytes)
    if words == 0:
        raise ValueError(f"buf size {nbytes} is not a positive multiple of 16 bytes")
    out = _out(out, "out", torch.int32, (words,), buf.device)
    st = lib.sv_read_probe(_ptr(buf), nbytes, _ptr(out), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_read_probe")
    return out


def sv_compact_accepted(src, dst, num_accepted, dst_start, path=None, *, out_status=None,
                        stream=None, want_status=True):
    """Accepted-path KV compaction through the C ABI.

    src uint8 [n, src_rows, row_bytes], dst uint8 [n, dst_rows, row_bytes] (modified in place),
    num_accepted and dst_start int32 [n], path int32 [n, path_len] or None (chains).  Returns a
    dict (status); the call is asynchronous.
    """
    lib = load()
    dev = src.device
    n, src_rows, row_bytes = src.shape
    _check(src, "src", torch.uint8, (n, src_rows, row_bytes), dev)
    _check(dst, "dst", torch.uint8, (n, dst.shape[1], row_bytes), dev)
    _check(num_accepted, "num_accepted", torch.int32, (n,), dev)
    _check(dst_start, "dst_start", torch.int32, (n,), dev)
    path_len = 0
    if path is not None:
        path_len = path.shape[1]
        _check(path, "path", torch.int32, (n, path_len), dev)
    if want_status or out_status is not None:
        out_status = _out(out_status, "out_status", torch.int32, (n,), dev)
    st = lib.sv_compact_accepted(_ptr(src), _ptr(dst), row_bytes, n, src_rows, dst.shape[1],
                                 _ptr(path), path_len, _ptr(num_accepted), _ptr(dst_start),
                                 _ptr(out_status), _stream(stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_compact_accepted")
    return {"status": out_status}


# ----------------------------------------------------------------------------- host arrays

def chain_to_device(batch, device="cuda"):
    """Copy a ChainBatch (numpy, from the inputs module) to device tensors."""
    dt = torch.bfloat16 if batch.dtype == "bf16" else torch.float32

    def logits(a):
        t = torch.from_numpy(a.view(np.int16) if batch.dtype == "bf16" else a)
        return (t.view(torch.bfloat16) if batch.dtype == "bf16" else t).to(device)

    return {
        "target": logits(batch.target), "draft": logits(batch.draft),
        "draft_tokens": torch.from_numpy(batch.draft_tokens).to(device),
        "uniforms": torch.from_numpy(batch.uniforms).to(device),
        "temperature": torch.from_numpy(batch.temperature).to(device),
        "dtype": dt,
    }


def greedy_to_device(batch, device="cuda"):
    """Copy a GreedyBatch to device tensors."""
    t = torch.from_numpy(batch.target.view(np.int16) if batch.dtype == "bf16" else batch.target)
    t = t.view(torch.bfloat16) if batch.dtype == "bf16" else t
    return {"target": t.to(device),
            "draft_tokens": torch.from_numpy(batch.draft_tokens).to(device)}


def sample_to_device(batch, device="cuda"):
    """Copy a SampleBatch to device tensors."""
    t = torch.from_numpy(batch.logits.view(np.int16) if batch.dtype == "bf16" else batch.logits)
    t = t.view(torch.bfloat16) if batch.dtype == "bf16" else t
    return {"logits": t.to(device),
            "temperature": torch.from_numpy(batch.temperature).to(device),
            "uniforms": torch.from_numpy(batch.uniforms).to(device)}


def kv_to_device(batch, device="cuda"):
    """Copy a KvBatch to device tensors (the destination starts as the batch's initial cache)."""
    return {"src": torch.from_numpy(batch.src).to(device),
            "dst": torch.from_numpy(batch.dst_init).to(device),
            "path": None if batch.paths is None else torch.from_numpy(batch.paths).to(device),
            "num_accepted": torch.from_numpy(batch.num_accepted).to(device),
            "dst_start": torch.from_numpy(batch.dst_start).to(device)}


def tree_to_device(batch, device="cuda"):
    t = torch.from_numpy(batch.logits.view(np.int16) if batch.dtype == "bf16" else batch.logits)
    t = t.view(torch.bfloat16) if batch.dtype == "bf16" else t
    return {
        "logits": t.to(device),
        "parents": torch.from_numpy(batch.parents).to(device),
        "node_tokens": torch.from_numpy(batch.node_tokens).to(device),
    }
