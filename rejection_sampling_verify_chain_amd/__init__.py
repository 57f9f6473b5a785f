"""specverify: the target-side verify step of speculative sampling on one MI355X.

The compute path is the HIP/gfx950 C-ABI library ``libspecverify.so`` (declared
in include/specverify.h); ``binding`` marshals torch device tensors into its
entry points.  ``inputs`` holds the seeded synthetic workloads.

The binding is imported lazily so that the input generators can be used on a
machine without the built library.
"""

import importlib

__all__ = ["sv_verify_chain", "sv_verify_tree", "binding", "inputs"]


def __getattr__(name):
    if name in ("binding", "inputs"):
        return importlib.import_module(f"{__name__}.{name}")
    if name in ("sv_verify_chain", "sv_verify_tree"):
        return getattr(importlib.import_module(f"{__name__}.binding"), name)
    raise AttributeError(name)
