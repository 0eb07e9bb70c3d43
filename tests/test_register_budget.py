"""The hot kernels keep every value in registers (host-only: hipcc remarks).

A kernel that spills VGPRs to scratch memory runs at a fraction of its speed
(the prefill MFMA kernel at 256 VGPRs per lane, two workgroups per CU, lost
about a quarter of its throughput to 43 spilled registers).  This compiles the
device code of each hot source for gfx950 and checks the compiler's resource
report: no VGPR spills and no scratch for the listed kernels.
"""
import os
import re
import subprocess

import pytest

from attention_paged_kv_write_amd import build

HOT = {
    "prefill.hip": ("prefill_mfma_kernel",),
    "decode.hip": ("decode_mfma_kernel", "decode_fp8_kernel", "decode_generic_kernel"),
    "reduce.hip": ("reduce_kernel", "reduce_small_kernel"),
    "kv_write.hip": ("",),
    "rope.hip": ("rope_kv_write_kernel",),
}


def resource_report(src):
    cmd = [build.HIPCC, *build.COMMON_FLAGS, "--offload-device-only", "-c", src, "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[bytes/lane\])?: (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("name", sorted(HOT))
def test_no_spills(name):
    report = resource_report(os.path.join(build.CSRC, name))
    checked = 0
    for fn, res in report.items():
        if not any(k in fn for k in HOT[name]):
            continue
        checked += 1
        assert res.get("VGPRs Spill", 0) == 0, f"{fn}: {res}"
        assert res.get("ScratchSize", 0) == 0, f"{fn}: {res}"
    assert checked > 0, f"no kernel of {name} in the report"
