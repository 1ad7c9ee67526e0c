"""The build's resource check: hipcc's per-kernel resource remarks are parsed,
written to _build/resources.txt, and any kernel that uses scratch memory (a
register spill) fails the build."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from block_scaled_fp4_mxfp4_amd import build  # noqa: E402

SAMPLE = """\
x.hip:10:1: remark: Function Name: _Z6kernelv [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     TotalSGPRs: 53 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     AGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     ScratchSize [bytes/lane]: 104 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     Occupancy [waves/SIMD]: 1 [-Rpass-analysis=kernel-resource-usage]
x.hip:10:1: remark:     VGPRs Spill: 25 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark: Function Name: _Z5otherv [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     VGPRs: 31 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:20:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
"""


def test_resource_remarks_are_parsed():
    rows = build.kernel_resources("x.hip", SAMPLE)
    assert rows == [("x.hip", "_Z6kernelv", 256, 256, 104, 25), ("x.hip", "_Z5otherv", 31, 0, 0, 0)]


def test_built_kernels_use_no_scratch():
    if not os.path.exists(build.RESOURCES):
        pytest.skip("library not built in this tree")
    lines = open(build.RESOURCES).read().splitlines()
    assert len(lines) >= 40, "every kernel of the library is listed"
    for line in lines:
        f = dict(p.split("=", 1) for p in line.split())
        assert f["scratch"] == "0" and f["spilled"] == "0", line
