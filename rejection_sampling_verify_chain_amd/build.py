"""Build libspecverify.so in-tree with hipcc for gfx950.

    python -m rejection_sampling_verify_chain_amd.build

Every call compiles from source (no staleness check): the library is small and a
full build takes seconds.  The result is written atomically next to this file.

Each .hip file is compiled in two passes of the HIP clang driver that hipcc wraps: the device
pass (gfx950 code object, bundled as a fat binary) carries the device-only flags, and the host
pass embeds that fat binary and registers its kernels.  Warnings are errors in every pass.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["sv_api.cpp", "sv_trace.cpp", "sv_argmax.hip", "sv_chain.hip", "sv_tree.hip",
           "sv_greedy.hip", "sv_kv.hip", "sv_probe.hip", "sv_noalloc.hip"]
ARCH = "gfx950"


def hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def hip_clang():
    """The HIP clang driver that hipcc wraps."""
    return os.environ.get("HIP_CLANG", "/opt/rocm/lib/llvm/bin/clang++")


def compile_flags():
    """Flags of every compile pass, host and device: warnings are errors."""
    return ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-ffp-contract=off", "-Wall",
            "-Wextra", "-Werror", "-I", INCLUDE, "-I", CSRC]


def device_flags():
    """Flags of the device pass only: packed fp32 instructions stay off (only scalar fp32 ops in
    device code).  The host pass does not know this target feature, so it never sees it."""
    return ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def compile_cmds(src, tmp, extra_flags=()):
    """Commands that turn one source into an object: a .hip file in two passes (the device code
    and its fat binary, then the host code that embeds it), a .cpp file in one host pass."""
    path = os.path.join(CSRC, src)
    obj = os.path.join(tmp, src + ".o")
    flags = [*compile_flags(), *extra_flags]
    if src.endswith(".hip"):
        fatbin = os.path.join(tmp, src + ".hipfb")
        return obj, [
            [hip_clang(), "-x", "hip", f"--offload-arch={ARCH}", "--cuda-device-only", *flags,
             *device_flags(), path, "-o", fatbin],
            [hip_clang(), "-x", "hip", f"--offload-arch={ARCH}", "--cuda-host-only", *flags,
             "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fatbin, "-c", path, "-o", obj],
        ]
    return obj, [[hip_clang(), "-x", "hip", "--cuda-host-only", *flags, "-c", path, "-o", obj]]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        # -Werror turns compiler diagnostics into errors; anything else a pass prints is shown.
        print(r.stderr, end="", file=sys.stderr, flush=True)
    return r


def build(verbose=False, out_path=LIB_PATH, extra_flags=()):
    """Compile every source and link the shared library; returns its path."""
    with tempfile.TemporaryDirectory(prefix="svbuild_") as tmp:
        objs, seqs = [], []
        for src in SOURCES:
            obj, cmds = compile_cmds(src, tmp, extra_flags)
            objs.append(obj)
            seqs.append(cmds)

        def run_seq(cmds):
            for c in cmds:
                _run(c, verbose)

        with ThreadPoolExecutor(len(seqs)) as ex:
            list(ex.map(run_seq, seqs))
        tmp_lib = os.path.join(tmp, LIB_NAME)
        _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp_lib],
             verbose)
        staged = out_path + ".tmp"
        with open(tmp_lib, "rb") as f, open(staged, "wb") as g:
            g.write(f.read())
        os.replace(staged, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
