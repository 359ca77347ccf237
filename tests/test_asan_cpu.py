"""The C interfaces' host code under AddressSanitizer (CPU only): the library's sources are built
once more with the sanitizer on their host side (gated_delta_linear_amd.build, sanitize=True),
and the CPU interface tests (tests/test_abi_cpu.py: argument checks, status strings, refusals
before any device work, the no-device path) run against that build in a child process with the
sanitizer runtime preloaded.  Any heap or stack error in the host code fails the run."""
import os
import shutil
import subprocess
import sys

import pytest

from gated_delta_linear_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _stale(lib: str) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC)] + [os.path.join(ROOT, "include", f)
                                                                           for f in os.listdir(os.path.join(ROOT, "include"))]
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.fixture(scope="module")
def asan_lib():
    rt = build.asan_runtime()
    if rt is None or not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("no hipcc or no clang AddressSanitizer runtime")
    if _stale(build.ASAN_LIB_PATH):
        build.build_library(sanitize=True)
    return build.ASAN_LIB_PATH, rt


def test_sanitized_build_is_instrumented(asan_lib):
    lib, _ = asan_lib
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms or "__asan_init" in syms


def test_interface_tests_pass_under_address_sanitizer(asan_lib):
    lib, rt = asan_lib
    env = dict(os.environ, LD_PRELOAD=rt, ARL2_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi_cpu.py"), "-q",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
