import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_collection_modifyitems(config, items):
    """GPU tests skip on a machine without a GPU; on a GPU machine they must run."""
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this machine")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session")
def gauss_b256():
    """The largest chain workload (B=256, gamma=7, V=152064, fp32, T in {0.6, 1.0}) and the
    oracle's result for every one of its sequences, built once for the tests that check the whole
    batch on each chain path."""
    from parity import chain_refs
    from rejection_sampling_verify_chain_amd import inputs as I
    b = I.chain_b256_v152064()
    return b, chain_refs(b)
