"""The multiply-shift divider of the transport kernels (qkvx::FastDiv, the
round-up method of Granlund and Montgomery, "Division by invariant integers
using multiplication", PLDI 1994) checked on the host against hardware
division over the range its header states (CPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is needed to compile the check")
def test_fastdiv_matches_division(tmp_path):
    exe = str(tmp_path / "fastdiv_check")
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROOT, 'head_exchange_amd', 'csrc')}",
           os.path.join(ROOT, "tests", "host", "fastdiv_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.startswith("ok "), out.stdout + out.stderr
