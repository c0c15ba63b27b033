"""The host library under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds ``libqkvx_sanitized.so`` (sanitizers on the host code only) and runs the
C-ABI tests of ``test_abi.py`` against it in a child process with the
sanitizer runtime preloaded: every validation path of the entry points (range,
alias, alignment and int32 checks, session bookkeeping) runs instrumented, and
any out-of-bounds access, use after free or undefined behaviour aborts the
child.  No GPU is touched (no call there reaches a kernel launch)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")),
                    reason="hipcc is needed to build the sanitized library")
def test_abi_tests_pass_under_asan_and_ubsan():
    from head_exchange_amd import build
    lib = build.build(sanitize=True)
    env = build.sanitizer_env()
    assert env["QKVX_LIB"] == lib
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-x", "-p", "no:cacheprovider"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    tail = (r.stdout[-2000:] + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail
