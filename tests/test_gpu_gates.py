"""GPU parity of the clean pass with alpha and beta from the gate projections
(arl2_commit_frame_gated) against the oracle's gate_projections + state write on the same
seeded hidden states and random-init gate weights.

Bar: max |err| / rms(output) <= 2e-2 and rel-Frobenius(S) <= 1e-3 after every frame.
"""
import numpy as np
import pytest
import torch

from synth import WORKLOADS, Workload
from tests.arl2_harness import OUT_TOL, STATE_TOL, log, run_stream

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _check(res, name):
    log(f"{name}: out_err {res['out_err']:.3e}, state_err max {max(res['state_err']):.3e}")
    assert res["out_err"] <= OUT_TOL, res["out_err"]
    assert max(res["state_err"]) <= STATE_TOL, res["state_err"]


SMALL = [  # (batch, heads, d, T, frames, denoise): odd H at d = 16 leaves H d off a 32-multiple
    (1, 1, 16, 5, 3, 1),
    (2, 3, 16, 37, 3, 1),
    (1, 2, 64, 100, 3, 1),
    (2, 5, 128, 129, 3, 1),
    (1, 12, 128, 300, 3, 1),
    (1, 40, 64, 70, 2, 1),
]


@pytest.mark.parametrize("B,H,d,T,frames,denoise", SMALL)
def test_gated_small_shapes(B, H, d, T, frames, denoise):
    w = Workload(f"gated_{B}_{H}_{d}_{T}", batch=B, heads=H, head_dim=d, tokens=T, frames=frames,
                 denoise_steps=denoise, seed=300 + T)
    _check(run_stream(w, gated=True), w.name)


def test_gated_dit480p_layer():
    """The DiT-layer shape, 6 frames of 4 + 1 passes, gates from 1536-wide hidden states."""
    w = WORKLOADS["dit480p"]
    _check(run_stream(w, frames=6, check_frames={0, 5}, reuse_denoise=True, gated=True), "gated dit480p")
