"""Every instantiated kernel of the library fits in registers: built for
gfx950 with the compiler's kernel-resource-usage remarks, no kernel uses
scratch memory (register spills or private arrays).  Also checks that the
launch plan's configurations all have a kernel (the count of instantiated
kernels does not drop silently)."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "positive_random_feature_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _resource_usage(source):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-c", os.path.join(CSRC, source), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    kernels = {}
    for block in r.stderr.split("Function Name: ")[1:]:
        name = block.split()[0]
        scratch = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", block)
        vgpr = re.search(r"VGPRs: (\d+)", block)
        kernels[name] = (int(scratch.group(1)), int(vgpr.group(1)))
    return kernels


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
@pytest.mark.parametrize("source,at_least", [("favor_kernels.hip", 150), ("hadamard_omega.hip", 4), ("givens_omega.hip", 1)])
def test_no_scratch(source, at_least):
    kernels = _resource_usage(source)
    assert len(kernels) >= at_least, len(kernels)
    spilling = {k: v for k, v in kernels.items() if v[0] != 0}
    print(f"{source}: {len(kernels)} kernels, max VGPRs {max(v[1] for v in kernels.values())}")
    assert not spilling, spilling
