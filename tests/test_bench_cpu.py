"""Host logic of bench.py that runs without a GPU: the oracle legs of every mode (on the tiny
workload), the algorithmic FLOP and byte counts, the kernel-source hash and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

import bench
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _check_leg(line, unit):
    assert line["kind"] == "oracle" and line["unit"] == unit
    assert line["value"] > 0 and line["cores"] >= 1
    assert line["sample"]


@pytest.mark.parametrize("gated,access", [(False, "frame"), (True, "frame"), (False, "token")])
def test_cpu_baseline_frames(gated, access):
    line = bench.cpu_baseline(WORKLOADS["tiny"], 0.05, gated=gated, access=access)
    _check_leg(line, "frame-tokens/s")


def test_cpu_baseline_recurrence_covers_the_stream():
    w = WORKLOADS["tiny"]
    line = bench.cpu_baseline_recurrence(w, 60.0)
    _check_leg(line, "state writes/s")
    assert f"frames 0..{w.frames - 1} of {w.frames}" in line["sample"]
    assert line["ms_per_state_write"] > 0


def test_cpu_baseline_softmax_and_backward():
    w = WORKLOADS["tiny"]
    sm = bench.cpu_baseline_softmax(w, 0.05)
    _check_leg(sm, "frame-tokens/s")
    assert len(sm["ms_per_frame"]) >= 1
    _check_leg(bench.cpu_baseline_backward(w, 0.05), "frame-tokens/s")


def test_algorithmic_counts_at_dit480p():
    """Per (stream, head): a pass 4 T^2 d + 2 T d^2 FLOPs; the state write alone reads K, V (bf16),
    beta, S_{N-1} and writes S_N (fp32), plus the maps phi_k, phi_v per head."""
    w = WORKLOADS["dit480p"]
    T, d, H = 1560, 128, 12
    assert bench.pass_flops(w) == H * (4 * T * T * d + 2 * T * d * d)
    assert bench.state_write_bytes(w) == H * (4 * T * d + 4 * T + 8 * d * d) + H * 4 * d * d
    assert abs(bench.pass_flops(w) / 1e9 - 15.565) < 1e-3


def test_kernel_source_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// a comment\nint f() { return 1; }  // trailing\n/* block\n comment */\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.hip"])
    h0 = bench.kernel_source_hash()
    src.write_text("// another comment\n\nint f() { return 1; }\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != h0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0 and "one GPU" in r.stderr
