"""GPU parity of the retained softmax layer (include/arl2_softmax.h) against its oracle, and its
cache protocol.

Bar: max |err| / rms(output) <= 2e-2 for every checked pass (the same output bar as the ARL2
layer's).  Inputs: the seeded synthetic streams of the ARL2 workloads (synth/).
"""
import numpy as np
import pytest
import torch

from gated_delta_linear_amd import SoftmaxLayer
from gated_delta_linear_amd.arl2 import ARL2_E_PROTOCOL, Arl2Error
from oracle import SoftmaxOracle
from synth import WORKLOADS, Workload, make_pass_inputs
from tests.arl2_harness import OUT_TOL, dev, log, out_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def run_stream(w, frames=None, rows=None, check=None, out_dtype=torch.float32, max_frames=None):
    """Run w's frames (denoising passes + clean pass) through the GPU layer and the oracle;
    returns the largest output error over the checked passes.  rows: query rows the oracle
    computes (all if None); check: frames whose passes are compared (all if None)."""
    frames = w.frames if frames is None else frames
    layer = SoftmaxLayer(w.batch, w.heads, w.head_dim, w.tokens, max_frames or frames, out_dtype=out_dtype)
    orc = SoftmaxOracle(w.head_dim)
    worst = 0.0
    for f in range(frames):
        for p in range(w.denoise_steps + 1):
            q, k, v = make_pass_inputs(w, f, p)
            qd, kd, vd = (dev(x, torch.bfloat16) for x in (q, k, v))
            clean = p == w.denoise_steps
            want_out = check is None or f in check
            if clean:
                got = layer.commit_frame(qd, kd, vd, want_output=want_out)
            else:
                got = layer.denoise_step(qd, kd, vd)
            if want_out:
                qs = q if rows is None else q[:, rows]
                ref = orc.attend(qs, k, v)
                g = got.float().cpu().numpy()
                g = g if rows is None else g[:, rows]
                worst = max(worst, out_err(g, ref))
            if clean:
                orc.commit_frame(q, k, v, want_output=False)
        assert layer.frame_index == f + 1
    torch.cuda.synchronize()
    layer.close()
    return worst


SMALL = [  # (batch, heads, d, T, frames, denoise)
    (1, 1, 16, 1, 3, 1),
    (1, 2, 16, 37, 3, 1),
    (1, 1, 64, 31, 4, 1),
    (2, 2, 64, 200, 3, 2),
    (1, 2, 128, 64, 3, 1),
    (1, 1, 128, 129, 4, 1),
    (2, 3, 128, 200, 3, 1),
    (1, 2, 128, 700, 3, 1),
]


@pytest.mark.parametrize("B,H,d,T,frames,denoise", SMALL)
def test_small_shapes(B, H, d, T, frames, denoise):
    w = Workload(f"kv_{B}_{H}_{d}_{T}", batch=B, heads=H, head_dim=d, tokens=T, frames=frames,
                 denoise_steps=denoise, seed=100 + T)
    err = run_stream(w)
    log(f"{w.name}: out_err {err:.3e}")
    assert err <= OUT_TOL, err


def test_bf16_output():
    w = Workload("kv_bf16out", batch=1, heads=2, head_dim=128, tokens=300, frames=3, denoise_steps=1, seed=21)
    err = run_stream(w, out_dtype=torch.bfloat16)
    log(f"{w.name}: out_err {err:.3e}")
    assert err <= OUT_TOL, err


def test_dit480p_layer_over_four_frames():
    """The DiT-layer shape (12 heads, d = 128, 1560 tokens), 4 frames of 4 + 1 passes: the clean
    passes of frames 0 and 3 checked on 96 sampled query rows (keys: 1560 and 6240)."""
    w = WORKLOADS["dit480p"]
    rows = np.random.default_rng(5).choice(w.tokens, 96, replace=False)
    err = run_stream(w, frames=4, rows=rows, check={0, 3})
    log(f"dit480p softmax layer: out_err {err:.3e}")
    assert err <= OUT_TOL, err


def test_denoising_passes_do_not_enter_the_cache():
    """Extra denoising passes with unrelated inputs leave the next frames' outputs bitwise equal."""
    w = Workload("kv_noise", batch=1, heads=2, head_dim=128, tokens=150, frames=3, denoise_steps=0, seed=31)
    noise = Workload("kv_noise2", batch=1, heads=2, head_dim=128, tokens=150, frames=3, denoise_steps=3, seed=32)
    outs = []
    for extra in (False, True):
        layer = SoftmaxLayer(w.batch, w.heads, w.head_dim, w.tokens, w.frames)
        res = []
        for f in range(w.frames):
            if extra:
                for p in range(3):
                    layer.denoise_step(*(dev(x, torch.bfloat16) for x in make_pass_inputs(noise, f, p)))
            q, k, v = (dev(x, torch.bfloat16) for x in make_pass_inputs(w, f, 0))
            res.append(layer.commit_frame(q, k, v).cpu())
        layer.close()
        outs.append(res)
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_runs_are_bitwise_reproducible():
    w = Workload("kv_repro", batch=2, heads=2, head_dim=64, tokens=333, frames=3, denoise_steps=1, seed=41)
    outs = []
    for _ in range(2):
        layer = SoftmaxLayer(w.batch, w.heads, w.head_dim, w.tokens, w.frames)
        res = []
        for f in range(w.frames):
            for p in range(w.denoise_steps + 1):
                q, k, v = (dev(x, torch.bfloat16) for x in make_pass_inputs(w, f, p))
                o = layer.denoise_step(q, k, v) if p < w.denoise_steps else layer.commit_frame(q, k, v)
                res.append(o.cpu())
        layer.close()
        outs.append(res)
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_full_cache_is_refused_and_reset_restarts():
    w = Workload("kv_full", batch=1, heads=1, head_dim=64, tokens=40, frames=2, denoise_steps=0, seed=51)
    layer = SoftmaxLayer(w.batch, w.heads, w.head_dim, w.tokens, 2)
    ins = [[dev(x, torch.bfloat16) for x in make_pass_inputs(w, f, 0)] for f in range(2)]
    first = layer.commit_frame(*ins[0]).cpu()
    layer.commit_frame(*ins[1])
    with pytest.raises(Arl2Error) as e:
        layer.denoise_step(*ins[0])
    assert e.value.status == ARL2_E_PROTOCOL
    assert layer.frame_index == 2
    layer.reset()
    assert layer.frame_index == 0
    assert torch.equal(layer.commit_frame(*ins[0]).cpu(), first)
    assert layer.device_bytes == 2 * 2 * w.tokens * w.heads * w.head_dim * 2
    layer.close()
