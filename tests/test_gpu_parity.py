"""GPU parity: libarl2 against the oracle on seeded streams (outputs and state).

Bar: max |err| / rms(output) <= 2e-2 and rel-Frobenius(S) <= 1e-3 after every frame.
"""
import numpy as np
import pytest
import torch

from gated_delta_linear_amd import Arl2Layer
from oracle import Arl2Oracle
from synth import WORKLOADS, Workload, make_gates, make_pass_inputs, make_phi
from tests.arl2_harness import OUT_TOL, STATE_TOL, dev, log, run_stream, state_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _check(res, name):
    log(f"{name}: out_err {res['out_err']:.3e}, state_err max {max(res['state_err']):.3e} "
        f"(last {res['state_err'][-1]:.3e}, |S| {res['state_norm']:.3e})")
    assert res["out_err"] <= OUT_TOL, res["out_err"]
    assert max(res["state_err"]) <= STATE_TOL, res["state_err"]


def test_tiny_workload():
    _check(run_stream(WORKLOADS["tiny"]), "tiny")


SMALL = [  # (batch, heads, d, T, frames, denoise)
    (1, 1, 16, 1, 2, 1),
    (1, 2, 16, 37, 3, 1),
    (1, 1, 64, 31, 2, 1),
    (2, 2, 64, 200, 3, 1),
    (1, 2, 128, 64, 2, 1),
    (1, 1, 128, 129, 2, 1),
    (2, 3, 128, 200, 3, 2),
    (1, 2, 128, 256, 2, 1),
    (1, 2, 128, 700, 2, 1),
]


@pytest.mark.parametrize("B,H,d,T,frames,denoise", SMALL)
def test_small_shapes(B, H, d, T, frames, denoise):
    w = Workload(f"small_{B}_{H}_{d}_{T}", batch=B, heads=H, head_dim=d, tokens=T, frames=frames,
                 denoise_steps=denoise, seed=7 + T)
    _check(run_stream(w), w.name)


def test_bf16_output():
    w = Workload("bf16out", batch=1, heads=2, head_dim=128, tokens=300, frames=3, denoise_steps=1, seed=11)
    _check(run_stream(w, out_dtype=torch.bfloat16), w.name)


def test_dit480p_layer_full_size():
    """1.3B DiT layer at 480p: 12 heads, d = 128, 1560 tokens, 21 frames of 4 + 1 passes."""
    w = WORKLOADS["dit480p"]
    res = run_stream(w, check_frames={0, 1, 20}, full_output_frames={0, 20}, reuse_denoise=True)
    _check(res, "dit480p")


def test_dit480p_literal_beta():
    """The same layer with beta = sigmoid(N(0, 1)) unscaled: the write is expansive and S grows
    by orders of magnitude per frame, but stays finite over 21 frames; relative errors hold."""
    w = WORKLOADS["dit480p"].with_(beta_mode="literal")
    res = run_stream(w, check_frames={0, 20}, reuse_denoise=True)
    assert np.isfinite(res["state_norm"]) and res["state_norm"] > 1e6
    _check(res, "dit480p_literal")


def test_chunked_generation_shapes():
    """Chunks of 3 latent frames (4680 tokens) as one unit, 4 streams; first 3 chunks."""
    w = WORKLOADS["chunked"]
    res = run_stream(w, frames=3, check_frames={0, 2}, sample_rows=48, reuse_denoise=True)
    _check(res, "chunked")


def test_long_stream_state_drift():
    """231 frames (about 921 video frames): state drift vs the oracle stays within the bar."""
    w = WORKLOADS["long_stream"]
    res = run_stream(w, check_frames={0, 1, 20, 114, 230}, sample_rows=48, reuse_denoise=True)
    for f in (20, 114, 230):
        log(f"long_stream: state_err after frame {f + 1}: {res['state_err'][f]:.3e}")
    _check(res, "long_stream")


def test_maximum_tokens_per_frame():
    """T = ARL2_MAX_TOKENS (2^20 tokens in one frame), one stream and head, d = 64: 8192 query
    tiles and 8192 state-write chunks per launch.  2 frames of a denoising pass + the clean pass;
    16 sampled output rows per pass and the full state after each frame."""
    from gated_delta_linear_amd.arl2 import ARL2_MAX_TOKENS
    w = Workload("max_tokens", batch=1, heads=1, head_dim=64, tokens=ARL2_MAX_TOKENS, frames=2, denoise_steps=1,
                 seed=71)
    res = run_stream(w, sample_rows=16, reuse_denoise=True)
    _check(res, "max_tokens")


def test_chunked_state_drift_77_chunks():
    """The chunked workload's whole stream: 77 commits of 4 streams x 12 heads x 4680 tokens (the
    clean passes' K, V and gates of 8 seeded chunks, cycled), state only.  S after chunks 1, 38 and
    77 against the oracle on streams 0 and 3, heads 0, 5 and 11 (every (stream, head) state is
    independent of the others)."""
    w = WORKLOADS["chunked"]
    ring = 8
    phis = make_phi(w)
    inputs = []
    for f in range(ring):
        _, k, v = make_pass_inputs(w, f, w.denoise_steps)
        beta, alpha = make_gates(w, f)
        inputs.append((k, v, beta, alpha))
    layer = Arl2Layer(*[dev(p, torch.bfloat16) for p in phis], batch=w.batch, tokens=w.tokens)
    bs, hs = [0, 3], [0, 5, 11]
    orcs = [Arl2Oracle(*[p[hs].astype(np.float64) for p in phis], batch=1) for _ in bs]
    staged = [tuple(dev(x, torch.bfloat16 if i < 2 else torch.float32) for i, x in enumerate(t)) for t in inputs]
    worst = 0.0
    for n in range(w.frames):
        k, v, beta, alpha = staged[n % ring]
        layer.commit_frame(None, k, v, beta, alpha, want_output=False)
        hk, hv, hb, ha = inputs[n % ring]
        for i, b in enumerate(bs):
            orcs[i].commit(None, hk[b:b + 1, :, hs], hv[b:b + 1, :, hs], hb[b:b + 1, :, hs], ha[b:b + 1, hs],
                           want_output=False)
        if n + 1 in (1, 38, 77):
            got = layer.state().cpu().numpy()
            err = max(state_err(got[b][hs], orcs[i].state[0]) for i, b in enumerate(bs))
            log(f"chunked: state_err after chunk {n + 1}: {err:.3e}")
            worst = max(worst, err)
    layer.close()
    assert worst <= STATE_TOL, worst

