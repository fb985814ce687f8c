"""Compile-time guard on the kernels' private memory: the device code of each
HIP source is compiled for gfx950 with the resource-usage remarks on, and no
kernel may use scratch (per-lane memory in HBM, from register spills or from
a private array the compiler could not keep in registers), except a few
spilled words in the prefill kernels' set-up.  Scratch in a decode loop costs
HBM traffic on every step.  No kernel is launched."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from unstructured_sparse_weight_amd import build as ub

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "unstructured_sparse_weight_amd", "csrc")
# Source -> most scratch bytes per lane any of its kernels may use.
LIMITS = {
    "usw_spmm.hip": 0,
    "usw_union.hip": 0,
    "usw_cbc.hip": 0,
    "usw_encode.hip": 0,
    "usw_probe.hip": 0,
    "usw_prefill.hip": 32,   # a few address registers spilled before the main loop
}


def hipcc_or_skip():
    try:
        return ub.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")


def resources(src):
    """{kernel: (scratch bytes per lane, spilled VGPRs)} from the remarks."""
    flags = [f for f in ub.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [hipcc_or_skip(), *flags, "--cuda-device-only", "-c", "-Rpass-analysis=kernel-resource-usage",
           "-I", ub.INCLUDE, "-I", CSRC, os.path.join(CSRC, src), "-o", os.devnull]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    out, name = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = [0, 0]
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            out[name][0] = int(m.group(1))
        m = re.search(r"VGPRs Spill: (\d+)", line)
        if m and name:
            out[name][1] = int(m.group(1))
    return out


@pytest.mark.slow
def test_no_kernel_uses_scratch():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    with ThreadPoolExecutor(max_workers=len(LIMITS)) as pool:
        found = dict(zip(LIMITS, pool.map(resources, LIMITS)))
    for src, kernels in found.items():
        assert kernels, f"no kernels reported for {src}"
        for k, (scratch, spills) in kernels.items():
            assert scratch <= LIMITS[src], f"{src}: {k} uses {scratch} bytes of scratch per lane"
            if LIMITS[src] == 0:
                assert spills == 0, f"{src}: {k} spills {spills} VGPRs"
