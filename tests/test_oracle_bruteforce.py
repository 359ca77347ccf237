"""Vectorised oracle against per-token / per-element scalar recomputation on tiny inputs."""
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import Arl2Oracle
from oracle.bruteforce import run_stream
from synth import WORKLOADS, make_gates, make_pass_inputs, make_phi


def _compare(phi_q, phi_k, phi_v, frames_in, batch, heads, atol=1e-12, rtol=0.0):
    orc = Arl2Oracle(phi_q, phi_k, phi_v, batch=batch)
    vec_out, vec_state = [], []
    for fr in frames_in:
        outs = []
        for p, (q, k, v) in enumerate(fr["passes"]):
            if p + 1 < len(fr["passes"]):
                outs.append(orc.denoise_step(q, k, v))
            else:
                outs.append(orc.commit(q, k, v, fr["beta"], fr["alpha"]))
        vec_out.append(outs)
        vec_state.append(orc.state.copy())
    for b in range(batch):
        for h in range(heads):
            frames = [{"passes": [(q[b, :, h], k[b, :, h], v[b, :, h]) for (q, k, v) in fr["passes"]],
                       "beta": fr["beta"][b, :, h], "alpha": fr["alpha"][b, h]} for fr in frames_in]
            bf_out, bf_state = run_stream(phi_q[h], phi_k[h], phi_v[h], frames)
            for f in range(len(frames_in)):
                for p in range(len(frames_in[f]["passes"])):
                    np.testing.assert_allclose(vec_out[f][p][b, :, h], np.array(bf_out[f][p]),
                                               rtol=rtol, atol=atol)
                np.testing.assert_allclose(vec_state[f][b, h], np.array(bf_state[f]), rtol=rtol, atol=atol)


def _frames_from_workload(w):
    frames = []
    for f in range(w.frames):
        passes = [make_pass_inputs(w, f, p) for p in range(w.denoise_steps + 1)]
        beta, alpha = make_gates(w, f)
        frames.append({"passes": [tuple(x.astype(np.float64) for x in ps) for ps in passes],
                       "beta": beta.astype(np.float64), "alpha": alpha.astype(np.float64)})
    return frames


def test_tiny_workload_fp32_draws():
    """The tiny workload exactly as specified (fp32 draws, d = 16, 4 frames x (2 + 1) passes)."""
    w = WORKLOADS["tiny"].with_(bf16_inputs=False)
    phis = [p.astype(np.float64) for p in make_phi(w)]
    _compare(*phis, _frames_from_workload(w), w.batch, w.heads)


def test_tiny_workload_bf16_values():
    """The same workload with the bf16-rounded values the GPU receives."""
    w = WORKLOADS["tiny"]
    phis = [p.astype(np.float64) for p in make_phi(w)]
    _compare(*phis, _frames_from_workload(w), w.batch, w.heads)


@settings(max_examples=25, deadline=None)
@given(batch=st.integers(1, 2), heads=st.integers(1, 3), tokens=st.integers(1, 24),
       d=st.sampled_from([1, 2, 4, 8]), frames=st.integers(1, 3), denoise=st.integers(0, 2),
       seed=st.integers(0, 2**31 - 1))
def test_random_tiny_shapes(batch, heads, tokens, d, frames, denoise, seed):
    rng = np.random.default_rng(seed)
    phis = [np.eye(d)[None] + 0.3 * rng.standard_normal((heads, d, d)) for _ in range(3)]
    frames_in = []
    for _ in range(frames):
        passes = [tuple(rng.standard_normal((batch, tokens, heads, d)) for _ in range(3))
                  for _ in range(denoise + 1)]
        frames_in.append({"passes": passes, "beta": rng.uniform(0, 1, (batch, tokens, heads)),
                          "alpha": rng.uniform(0, 1, (batch, heads))})
    _compare(*phis, frames_in, batch, heads, atol=1e-11, rtol=1e-10)
