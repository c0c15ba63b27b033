"""Build the gfx950 shared library ``libqkvx.so`` in-tree with hipcc.

Run ``python -m head_exchange_amd.build``.  The
library is written next to this file so that it travels with the source tree.

``python -m head_exchange_amd.build --sanitize`` builds ``libqkvx_sanitized.so``
instead: the same sources with AddressSanitizer and UndefinedBehaviorSanitizer
on the host code only (the device code is built as usual), for running the CPU
tests of the host library (argument validation, range and alias checks) under
the sanitizers; ``sanitizer_env()`` gives the environment such a run needs.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqkvx.so")
LIB_SANITIZED = os.path.join(HERE, "libqkvx_sanitized.so")
OBJDIR = os.path.join(ROOT, "_build")
SOURCES = ["qkvx_host.cpp", "qkvx_fused.hip", "qkvx_transport.hip", "qkvx_ready.hip"]

ARCH = "gfx950"
FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed-fp32 forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
    # per-kernel register and scratch figures, checked after each compile
    "-Rpass-analysis=kernel-resource-usage",
]

_REMARK = re.compile(r"remark: +(Function Name|ScratchSize \[bytes/lane\]|VGPRs|AGPRs): (\S+)")


def resource_usage(stderr: str) -> dict:
    """Per-kernel {"VGPRs", "AGPRs", "ScratchSize"} from the compiler's
    kernel-resource-usage remarks."""
    usage, name = {}, None
    for key, val in _REMARK.findall(stderr):
        if key == "Function Name":
            name = val
            usage[name] = {}
        elif name is not None:
            usage[name][key.split()[0]] = int(val)
    return usage


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqkvx.so)")


# host-side sanitizers only: each option applies to the host compilation
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
            "-g"]


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    suffix = "_sanitized" if sanitize else ""
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [hipcc()] + FLAGS + (SANITIZE if sanitize else []) + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    # Every kernel's register plan leaves no spills: the fused kernel holds all
    # 256 AGPRs of accumulators and ~200 VGPRs of operand fragments, and a
    # compiler that spilled there would run the main loop through scratch
    # memory, correct but far slower, without any other sign.
    spills = {k: u["ScratchSize"] for k, u in resource_usage(r.stderr).items()
              if u.get("ScratchSize", 0) > 0}
    if spills:
        raise RuntimeError(f"{src}: kernels spill registers to scratch memory "
                           f"(bytes per lane): {spills}")
    if verbose:
        rest = "\n".join(l for l in r.stderr.splitlines() if "kernel-resource-usage" not in l)
        if rest.strip():
            print(rest, file=sys.stderr)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP source for gfx950 and link ``libqkvx.so`` (or, with
    ``sanitize``, ``libqkvx_sanitized.so``); returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), SOURCES))
    lib = LIB_SANITIZED if sanitize else LIB
    tmp = lib + ".tmp"
    link_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-shared-libsan"] if sanitize else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + link_san + ["-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def sanitizer_env() -> dict:
    """Environment for running the sanitized library inside an uninstrumented
    Python: the compiler's AddressSanitizer runtime preloaded, leak checking off
    (the interpreter's own allocations are not ours), the binding pointed at
    ``libqkvx_sanitized.so``."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    rt = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True, check=True).stdout.strip()
    env = dict(os.environ)
    env.update({"LD_PRELOAD": rt, "QKVX_LIB": LIB_SANITIZED,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    return env


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
