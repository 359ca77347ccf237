"""The allocation-free clean pass (arl2_commit_frame_noalloc, include/arl2.h) through the C
interface, against the layer's arl2_commit_frame on the same inputs and state.

Both run the same kernels in the same order, so outputs and states must agree bitwise; the
first stream is also checked against the oracle (the layer's bars: max |err| / rms(output) <=
2e-2, rel-Frobenius(S) <= 1e-3).  Calls come in a row on one stream, each reusing the library's
device array: the 1.3B DiT layer shape over two frames, then smaller frames (fewer heads, fewer
tokens, d = 64 and d = 16), so that a later call that read what an earlier, larger one left in
the array would show.  Sizes beyond the array are refused.
"""
import numpy as np
import pytest
import torch

from gated_delta_linear_amd.arl2 import ARL2_E_UNSUPPORTED, Arl2Error, Arl2Layer, commit_frame_noalloc
from oracle import Arl2Oracle
from synth import Workload, make_gates, make_pass_inputs, make_phi
from tests.arl2_harness import OUT_TOL, STATE_TOL, dev, log, out_err, state_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _stream_pair(w, frames, with_oracle=False, out_dtype=torch.float32):
    phis = make_phi(w)
    phis_d = [dev(p, torch.bfloat16) for p in phis]
    layer = Arl2Layer(*phis_d, batch=w.batch, tokens=w.tokens, out_dtype=out_dtype)
    orc = Arl2Oracle(*[p.astype(np.float64) for p in phis], batch=w.batch) if with_oracle else None
    state = torch.zeros(layer.state_shape, dtype=torch.float32, device="cuda")
    worst_o = worst_s = 0.0
    try:
        for f in range(frames):
            q, k, v = make_pass_inputs(w, f, w.denoise_steps)
            beta, alpha = make_gates(w, f)
            qd, kd, vd = (dev(x, torch.bfloat16) for x in (q, k, v))
            bd, ad = dev(beta, torch.float32), dev(alpha, torch.float32)
            want = layer.commit_frame(qd, kd, vd, bd, ad)
            got = torch.empty_like(want)
            commit_frame_noalloc(*phis_d, state, qd, kd, vd, bd, ad, out=got)
            assert torch.equal(got, want), f
            assert torch.equal(state, layer.state()), f
            if orc is not None:
                ref = orc.commit(q, k, v, beta, alpha)
                worst_o = max(worst_o, out_err(got.double().cpu().numpy(), ref))
                worst_s = max(worst_s, state_err(state.double().cpu().numpy(), orc.state))
        # the state write alone (no output)
        q, k, v = make_pass_inputs(w, frames, w.denoise_steps)
        beta, alpha = make_gates(w, frames)
        kd, vd, bd, ad = dev(k, torch.bfloat16), dev(v, torch.bfloat16), dev(beta, torch.float32), dev(alpha, torch.float32)
        layer.commit_frame(None, kd, vd, bd, ad, want_output=False)
        commit_frame_noalloc(*phis_d, state, None, kd, vd, bd, ad)
        assert torch.equal(state, layer.state())
    finally:
        torch.cuda.synchronize()
        layer.close()
    return worst_o, worst_s


def test_noalloc_matches_layer_then_smaller_frames():
    cases = [
        (Workload("na_dit", batch=1, heads=12, head_dim=128, tokens=1560, frames=2, denoise_steps=4, seed=31), 2, False),
        (Workload("na_small", batch=2, heads=3, head_dim=128, tokens=300, frames=2, denoise_steps=1, seed=32), 2, True),
        (Workload("na_d64", batch=1, heads=2, head_dim=64, tokens=129, frames=2, denoise_steps=1, seed=33), 2, True),
        (Workload("na_d16", batch=1, heads=1, head_dim=16, tokens=37, frames=3, denoise_steps=1, seed=34), 3, True),
    ]
    for w, frames, with_oracle in cases:
        o, s = _stream_pair(w, frames, with_oracle)
        log(f"{w.name}: bitwise equal to the layer; oracle out_err {o:.3e}, state_err {s:.3e}")
        assert o <= OUT_TOL and s <= STATE_TOL, (w.name, o, s)


def test_noalloc_bf16_output():
    w = Workload("na_bf16", batch=1, heads=2, head_dim=128, tokens=200, frames=2, denoise_steps=1, seed=35)
    _stream_pair(w, 2, out_dtype=torch.bfloat16)


def test_noalloc_refuses_frames_beyond_its_array():
    B, H, d, T = 4, 12, 128, 4680  # the chunked workload: about 120 MB of partial sums
    phi = torch.zeros((H, d, d), dtype=torch.bfloat16, device="cuda")
    state = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    x = torch.zeros((B, T, H, d), dtype=torch.bfloat16, device="cuda")
    beta = torch.zeros((B, T, H), dtype=torch.float32, device="cuda")
    alpha = torch.ones((B, H), dtype=torch.float32, device="cuda")
    with pytest.raises(Arl2Error) as e:
        commit_frame_noalloc(phi, phi, phi, state, x, x, x, beta, alpha)
    assert e.value.status == ARL2_E_UNSUPPORTED and "scratch" in str(e.value)
