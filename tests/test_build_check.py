"""The build's register-spill check: the compiler's kernel-resource-usage
remarks are parsed per kernel, and a kernel with scratch memory is reported."""
import os
import subprocess

import pytest

from head_exchange_amd import build

KERNEL = r"""
#include <hip/hip_runtime.h>
__global__ void plain(float* o) { o[threadIdx.x] = 1.0f; }
__global__ void private_array(float* o, int i) {
    float a[256];
    for (int k = 0; k < 256; ++k) a[k] = o[k];
    o[threadIdx.x] = a[(i + threadIdx.x) & 255];
}
"""


def test_remarks_parse():
    text = "\n".join([
        "f.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "f.hip:1:1: remark:     VGPRs: 254 [-Rpass-analysis=kernel-resource-usage]",
        "f.hip:1:1: remark:     AGPRs: 256 [-Rpass-analysis=kernel-resource-usage]",
        "f.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "f.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "f.hip:9:1: remark:     VGPRs: 12 [-Rpass-analysis=kernel-resource-usage]",
        "f.hip:9:1: remark:     ScratchSize [bytes/lane]: 1024 [-Rpass-analysis=kernel-resource-usage]",
    ])
    u = build.resource_usage(text)
    assert u == {"kern_a": {"VGPRs": 254, "AGPRs": 256, "ScratchSize": 0},
                 "kern_b": {"VGPRs": 12, "ScratchSize": 1024}}


def test_compiler_reports_scratch(tmp_path):
    try:
        cc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    src = tmp_path / "k.hip"
    src.write_text(KERNEL)
    flags = [f for f in build.FLAGS if not f.startswith("-I")]
    r = subprocess.run([cc] + flags + ["--cuda-device-only", "-c", str(src), "-o",
                                       str(tmp_path / "k.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    u = build.resource_usage(r.stderr)
    plain = [v for k, v in u.items() if "plain" in k]
    priv = [v for k, v in u.items() if "private_array" in k]
    assert plain and plain[0]["ScratchSize"] == 0
    assert priv and priv[0]["ScratchSize"] > 0, u
