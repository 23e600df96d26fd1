"""Builds libpa.so in-tree with hipcc for gfx950.

Usage: python -m paged_kv_cache_65_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
TRACE_LIB = os.path.join(HERE, "libpa_trace.so")  # diagnostic build with per-wave timestamps
SOURCES = ["pa_kernels.hip", "pa_pool.cpp", "pa_error.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # packed fp32 instructions stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in VGPRs: the softmax rescale then works on them in place
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False, extra_flags=(), trace: bool = False) -> str:
    """Builds libpa.so; with trace=True the diagnostic libpa_trace.so instead
    (-DPA_TRACE: the balanced and extend kernels record per-wave timestamps)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    out = TRACE_LIB if trace else LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(["-DPA_TRACE"] if trace else []), *extra_flags, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if errs.strip() and verbose:
        print(errs, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, trace="--trace" in sys.argv[1:]))
