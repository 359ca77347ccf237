"""GPU parity of the token-level (sequential) access variant (arl2_denoise_step_seq /
arl2_commit_frame_seq) against its oracle (oracle/seq_oracle.py), and the A/B property that
separates it from frame-level access.

Bar: max |err| / rms(output) <= 2e-2 on every pass and rel-Frobenius(S) <= 1e-3 after every frame.
"""
import numpy as np
import pytest
import torch

from gated_delta_linear_amd import Arl2Layer
from oracle import Arl2SeqOracle
from synth import WORKLOADS, Workload, make_gates, make_pass_inputs, make_phi
from tests.arl2_harness import OUT_TOL, STATE_TOL, dev, log, out_err, state_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def run_seq(w, frames=None, rows=None, check=None):
    frames = w.frames if frames is None else frames
    phis = make_phi(w)
    layer = Arl2Layer(*[dev(p, torch.bfloat16) for p in phis], batch=w.batch, tokens=w.tokens, access="token")
    orc = Arl2SeqOracle(*[p.astype(np.float64) for p in phis], batch=w.batch)
    worst, serr = 0.0, []
    try:
        for f in range(frames):
            beta, alpha = make_gates(w, f)
            bd, ad = dev(beta, torch.float32), dev(alpha, torch.float32)
            for p in range(w.denoise_steps + 1):
                q, k, v = make_pass_inputs(w, f, p)
                qd, kd, vd = (dev(x, torch.bfloat16) for x in (q, k, v))
                clean = p == w.denoise_steps
                if clean:
                    got = layer.commit_frame_seq(qd, kd, vd, bd, ad)
                    want = orc.commit(q, k, v, beta, alpha)
                else:
                    got = layer.denoise_step_seq(qd, kd, vd, bd)
                    want = orc.denoise_step(q, k, v, beta)
                if check is None or f in check:
                    g = got.double().cpu().numpy()
                    if rows is not None:
                        g, want = g[:, rows], want[:, rows]
                    worst = max(worst, out_err(g, want))
            serr.append(state_err(layer.state().double().cpu().numpy(), orc.state))
        assert layer.frame_index == frames
    finally:
        layer.close()
    return worst, serr


SMALL = [  # (batch, heads, d, T, frames, denoise)
    (1, 1, 64, 1, 3, 1),
    (1, 2, 64, 37, 3, 1),
    (2, 2, 64, 64, 3, 1),
    (1, 1, 128, 65, 3, 1),
    (2, 3, 128, 200, 3, 2),
    (1, 2, 128, 333, 3, 1),
]


@pytest.mark.parametrize("B,H,d,T,frames,denoise", SMALL)
def test_seq_small_shapes(B, H, d, T, frames, denoise):
    w = Workload(f"seq_{B}_{H}_{d}_{T}", batch=B, heads=H, head_dim=d, tokens=T, frames=frames,
                 denoise_steps=denoise, seed=500 + T)
    err, serr = run_seq(w)
    log(f"{w.name}: out_err {err:.3e}, state_err max {max(serr):.3e}")
    assert err <= OUT_TOL, err
    assert max(serr) <= STATE_TOL, serr


def test_seq_dit480p_layer():
    """The DiT-layer shape (12 heads, d = 128, 1560 tokens: 25 chunks), 3 frames of 1 + 1 passes."""
    w = WORKLOADS["dit480p"].with_(denoise_steps=1)
    err, serr = run_seq(w, frames=3)
    log(f"seq dit480p: out_err {err:.3e}, state_err max {max(serr):.3e}")
    assert err <= OUT_TOL, err
    assert max(serr) <= STATE_TOL, serr


def test_seq_is_not_permutation_equivariant_and_frame_level_is():
    """Permuting a frame's tokens permutes the frame-level layer's outputs, not the token-level
    layer's: the asymmetry the pages avoid, seen on the GPU."""
    w = Workload("seq_perm", batch=1, heads=2, head_dim=128, tokens=96, frames=2, denoise_steps=0, seed=77)
    perm = np.random.default_rng(1).permutation(w.tokens)
    phis = [dev(p, torch.bfloat16) for p in make_phi(w)]
    res = {}
    for access in ("frame", "token"):
        outs = []
        for pm in (None, perm):
            layer = Arl2Layer(*phis, batch=1, tokens=w.tokens, access=access)
            for f in range(2):
                q, k, v = make_pass_inputs(w, f, 0)
                beta, alpha = make_gates(w, f)
                if pm is not None and f == 1:
                    q, k, v, beta = q[:, pm], k[:, pm], v[:, pm], beta[:, pm]
                args = [dev(x, torch.bfloat16) for x in (q, k, v)]
                bd, ad = dev(beta, torch.float32), dev(alpha, torch.float32)
                o = layer.commit_frame(*args, bd, ad) if access == "frame" else layer.commit_frame_seq(*args, bd, ad)
            outs.append(o.double().cpu().numpy())
            layer.close()
        base, permuted = outs
        res[access] = np.abs(permuted - base[:, perm]).max() / np.sqrt(np.mean(base ** 2))
    log(f"permutation: frame-level {res['frame']:.2e}, token-level {res['token']:.2e}")
    assert res["frame"] < 1e-3
    assert res["token"] > 1e-2


def test_access_modes_are_not_mixed():
    from gated_delta_linear_amd.arl2 import ARL2_E_INVALID_ARG, Arl2Error
    w = Workload("seq_mix", batch=1, heads=1, head_dim=64, tokens=32, frames=1, denoise_steps=0, seed=3)
    phis = [dev(p, torch.bfloat16) for p in make_phi(w)]
    q, k, v = (dev(x, torch.bfloat16) for x in make_pass_inputs(w, 0, 0))
    beta, alpha = (dev(x, torch.float32) for x in make_gates(w, 0))
    tok = Arl2Layer(*phis, batch=1, tokens=32, access="token")
    with pytest.raises(Arl2Error) as e:
        tok.denoise_step(q, k, v)
    assert e.value.status == ARL2_E_INVALID_ARG
    tok.close()
    frm = Arl2Layer(*phis, batch=1, tokens=32)
    with pytest.raises(Arl2Error) as e:
        frm.commit_frame_seq(q, k, v, beta, alpha)
    assert e.value.status == ARL2_E_INVALID_ARG
    frm.close()
