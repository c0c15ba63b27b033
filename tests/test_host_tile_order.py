"""The fused kernel's tile order (qkvx::TileOrder, the code the kernel runs) and
its tile-claim protocol, checked on the host: every tile is named by exactly
one queue position for every order, queue count and grid shape; simulated
random interleavings of the claiming workgroups run every tile exactly once;
the band counts of the benchmark shapes (CPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is needed to compile the check")
def test_tile_order_and_claims_cover_every_tile(tmp_path):
    exe = str(tmp_path / "tile_order_check")
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROOT, 'head_exchange_amd', 'csrc')}",
           os.path.join(ROOT, "tests", "host", "tile_order_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.startswith("ok "), out.stdout + out.stderr
