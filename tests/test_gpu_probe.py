"""GPU check of the streaming-read ceiling probe (measurement support): every workgroup's output
word is the XOR of the 32-bit words it read, so a dropped or misplaced load shows."""

import numpy as np
import pytest
import torch

from rejection_sampling_verify_chain_amd import binding as BD

pytestmark = pytest.mark.gpu

GROUP_WORDS = 128 * 1024 // 4  # 32-bit words one probe workgroup reads


@pytest.mark.parametrize("nbytes", [16, 4096, 131072, 3 * 131072 + 48, 1 << 22])
def test_read_probe_xor(nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = BD.sv_read_probe(buf)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    want = np.array([np.bitwise_xor.reduce(host[i:i + GROUP_WORDS])
                     for i in range(0, len(host), GROUP_WORDS)], dtype=np.uint32)
    assert np.array_equal(got, want)
