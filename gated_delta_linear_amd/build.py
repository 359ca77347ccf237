"""Build libarl2.so (HIP kernels + C interface) for gfx950 with hipcc, in the package directory.

Usage: python -m gated_delta_linear_amd.build [-v]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libarl2.so")
SOURCES = ["arl2_fwd.hip", "arl2_commit.hip", "arl2_kvcache.hip", "arl2_gates.hip", "arl2_seq.hip", "arl2_bwd.hip",
           "arl2_host.cpp", "arl2_softmax_host.cpp", "arl2_bwd_host.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libarl2.so)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-function",
        # no packed fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source into libarl2.so; always recompiles."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *compile_flags(), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
