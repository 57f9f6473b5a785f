"""Build libspecverify.so in-tree with hipcc for gfx950.

    python -m rejection_sampling_verify_chain_amd.build

Every call compiles from source (no staleness check): the library is small and a
full build takes seconds.  The result is written atomically next to this file.
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


def compile_flags():
    return [
        "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-ffp-contract=off", "-Wall",
        f"--offload-arch={ARCH}",
        # Packed fp32 instructions stay off (only scalar fp32 ops in device code).
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose=False, out_path=LIB_PATH, extra_flags=()):
    """Compile every source and link the shared library; returns its path."""
    with tempfile.TemporaryDirectory(prefix="svbuild_") as tmp:
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            cmds.append([hipcc(), *compile_flags(), *extra_flags, "-c",
                         os.path.join(CSRC, src), "-o", obj])
        with ThreadPoolExecutor(len(cmds)) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
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
