"""The build keeps packed fp32 instructions out of the device code (CPU only).

build.py passes the target-feature switch that turns them off to the device pass only (the host
pass does not know it).  This test compiles device assembly with the build's own flags and
checks that no packed fp32 add, multiply or FMA appears, in the library's largest translation
unit and in a small float2 kernel that the compiler packs when the switch is missing (the
control, which shows the check can fail).
"""

import os
import re
import shutil
import subprocess

import pytest

from rejection_sampling_verify_chain_amd import build as BLD

PACKED_F32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
FLOAT2_KERNEL = """
#include <hip/hip_runtime.h>
__global__ void k(float2* a, float2 b) {
  const int i = threadIdx.x;
  a[i] = make_float2(a[i].x * b.x + 1.0f, a[i].y * b.y + 2.0f);
}
"""

pytestmark = pytest.mark.skipif(not os.path.exists(BLD.hip_clang()), reason="needs HIP clang")


def device_asm(src, tmp_path, device_flags=True):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [BLD.hip_clang(), "-x", "hip", f"--offload-arch={BLD.ARCH}", "--cuda-device-only",
           *BLD.compile_flags(), *(BLD.device_flags() if device_flags else []), "-S", src,
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return out.read_text()


def test_control_kernel_packs_without_the_switch(tmp_path):
    src = tmp_path / "float2.hip"
    src.write_text(FLOAT2_KERNEL)
    assert PACKED_F32.search(device_asm(str(src), tmp_path, device_flags=False))
    assert not PACKED_F32.search(device_asm(str(src), tmp_path, device_flags=True))


@pytest.mark.parametrize("name", ["sv_chain.hip", "sv_argmax.hip"])
def test_library_device_code_has_no_packed_fp32(name, tmp_path):
    asm = device_asm(os.path.join(BLD.CSRC, name), tmp_path)
    assert "amdgcn" in asm or ".amdhsa" in asm
    hits = PACKED_F32.findall(asm)
    assert not hits, f"{name}: {len(hits)} packed fp32 instructions"


def test_host_pass_never_sees_the_device_switch(tmp_path):
    for src in BLD.SOURCES:
        _, cmds = BLD.compile_cmds(src, str(tmp_path))
        for c in cmds:
            if "--cuda-device-only" not in c:
                assert "-packed-fp32-ops" not in c, (src, c)
