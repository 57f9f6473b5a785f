"""Host-side parts of bench.py that need no GPU: the one-GPU guard and the CPU baseline legs."""

import os
import subprocess
import sys

import bench
from rejection_sampling_verify_chain_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_legs():
    chain = I.chain_b1_v1000()
    tree = I.tree_random(5, 2, 16, 500, "bf16")
    r = bench.cpu_baseline(chain, tree, None, None, None, None, 0.6)
    assert r["kind"] == "oracle" and r["unit"] == "rows/s"
    assert r["value"] > 0 and r["single_core_value"] > 0 and r["cores"] >= 1
    assert "forked worker processes" in r["sample"] and "one process" in r["single_core_sample"]
