"""GPU parity of sv_compact_accepted against the oracle (through the C ABI)."""

import numpy as np
import pytest
import torch

from parity import check_kv
from rejection_sampling_verify_chain_amd import binding as BD
from rejection_sampling_verify_chain_amd import inputs as I

pytestmark = pytest.mark.gpu


def run_kv(batch):
    d = BD.kv_to_device(batch)
    out = BD.sv_compact_accepted(d["src"], d["dst"], d["num_accepted"], d["dst_start"],
                                 d["path"])
    torch.cuda.synchronize()
    return d["dst"].cpu().numpy(), out["status"].cpu().numpy()


@pytest.mark.parametrize("name", sorted(I.KV_WORKLOADS))
def test_full_size_workloads(name):
    b = I.KV_WORKLOADS[name]()
    check_kv(b, *run_kv(b))
    print(f"[parity] {name}: rows moved {b.moved_rows}", flush=True)


@pytest.mark.parametrize("row_bytes", [1, 3, 16, 1000, 1028, 4096, 16400, 65536 + 4])
def test_row_widths_tree_and_chain(row_bytes):
    tree = I.kv_tree_paths(row_bytes, 9, 30, row_bytes, dst_rows=20)
    check_kv(tree, *run_kv(tree))
    chain = I.kv_chain(row_bytes + 1, 7, 5, row_bytes, dst_rows=9)
    check_kv(chain, *run_kv(chain))


def test_bad_indices_copy_nothing():
    b = I.kv_tree_paths(50, 8, 20, 256, dst_rows=12)
    b.paths[1, 1] = 20                      # node id outside the block
    b.num_accepted[2] = 20                  # more than the path length allows
    b.dst_start[3] = 12 - b.num_accepted[3]  # one row past the cache's end
    b.num_accepted[4] = -1
    dst, st = run_kv(b)
    check_kv(b, dst, st)
    for t in (1, 2, 3, 4):
        assert st[t] == BD.ROW_BAD_INDEX and np.array_equal(dst[t], b.dst_init[t])


def test_after_tree_verification_on_device():
    # Verify, then compact with the verify's device outputs: the cache rows read back as the
    # KV rows of the root and the accepted nodes.
    tree = I.tree_random(51, 12, 40, 3000, "bf16", boost=20.0, boost_prob=1.0)
    t = BD.tree_to_device(tree)
    vo = BD.sv_verify_tree(t["logits"], t["parents"], t["node_tokens"])
    kv = I.kv_tree_paths(52, 12, 40, 512, dst_rows=48)
    d = BD.kv_to_device(kv)
    start = torch.zeros(12, dtype=torch.int32, device=d["src"].device)
    out = BD.sv_compact_accepted(d["src"], d["dst"], vo["num_accepted"], start, vo["path"])
    torch.cuda.synchronize()
    path = vo["path"].cpu().numpy()
    k = vo["num_accepted"].cpu().numpy()
    dst = d["dst"].cpu().numpy()
    assert not out["status"].cpu().numpy().any() and k.max() >= 3
    for i in range(12):
        for j in range(k[i] + 1):
            assert np.array_equal(dst[i, j], kv.src[i, path[i, j]])
        assert np.array_equal(dst[i, k[i] + 1:], kv.dst_init[i, k[i] + 1:])
