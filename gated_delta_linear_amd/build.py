"""Build libarl2.so (HIP kernels + C interface) for gfx950 with hipcc, in the package directory.

Usage: python -m gated_delta_linear_amd.build [-v] [--asan]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libarl2.so")
SOURCES = ["arl2_fwd.hip", "arl2_commit.hip", "arl2_kvcache.hip", "arl2_gates.hip", "arl2_seq.hip", "arl2_bwd.hip", "arl2_convert.hip", "arl2_noalloc.hip", "arl2_linear.hip",
           "arl2_host.cpp", "arl2_softmax_host.cpp", "arl2_bwd_host.cpp", "arl2_linear_host.cpp"]
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


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{msgs}")
    return msgs


ASAN_LIB_PATH = os.path.join(PKG_DIR, "_build", "asan", "libarl2.so")
# host code only: the sanitizer instruments the CPU side of every source (the interface's
# argument checks, the layer objects), never device code
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str | None:
    """The clang AddressSanitizer runtime a process must preload to load the sanitized library."""
    import glob

    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def build_library(verbose: bool = False, jobs: int | None = None, sanitize: bool = False) -> str:
    """Compile every HIP source into libarl2.so; always recompiles (one object per source, in
    parallel, under _build/, then one link).  sanitize=True builds the AddressSanitizer variant
    of the host code into _build/asan/libarl2.so instead (for the CPU interface tests)."""
    from concurrent.futures import ThreadPoolExecutor

    obj_dir = os.path.join(PKG_DIR, "_build", "asan") if sanitize else os.path.join(PKG_DIR, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    flags = [f for f in compile_flags() if f != "-shared"] + (ASAN_FLAGS if sanitize else [])
    cmds = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        cmds.append((obj, [hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj]))
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        for (obj, cmd), msgs in zip(cmds, pool.map(lambda c: _run(c[1]), cmds)):
            if verbose:
                print(" ".join(cmd), flush=True)
                if msgs.strip():
                    print(msgs)
    lib_path = ASAN_LIB_PATH if sanitize else LIB_PATH
    tmp = lib_path + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", *(ASAN_FLAGS if sanitize else []),
            *[o for o, _ in cmds], "-o", tmp]
    msgs = _run(link)
    if verbose:
        print(" ".join(link), flush=True)
        if msgs.strip():
            print(msgs)
    os.replace(tmp, lib_path)
    return lib_path


PROBE_SRC = os.path.join(CSRC, "probe_mfma_rate.hip")
PROBE_PATH = os.path.join(PKG_DIR, "probe_mfma_rate")


def build_probe(verbose: bool = False) -> str:
    """Compile the sustained-MFMA-rate probe (a standalone measurement program, not part of
    libarl2.so) into the package directory, beside the library."""
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", PROBE_SRC, "-o", PROBE_PATH + ".tmp"]
    msgs = _run(cmd)
    if verbose:
        print(" ".join(cmd), flush=True)
        if msgs.strip():
            print(msgs)
    os.replace(PROBE_PATH + ".tmp", PROBE_PATH)
    return PROBE_PATH


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv, sanitize="--asan" in sys.argv))
    if "--asan" not in sys.argv:
        print(build_probe(verbose="-v" in sys.argv))
