"""GPU protocol tests: the query-many / commit-once rules hold bitwise on the device.

Pins the library to the statements of "Attend Locally, Remember Linearly" (gist.science
technical summary, section 2.2): denoising passes never write the state, the clean pass
writes it once, and all tokens of a frame read the same pre-update state.
"""
import numpy as np
import pytest
import torch

from gated_delta_linear_amd import Arl2Error, Arl2Layer
from synth import Workload, make_gates, make_pass_inputs, make_phi
from tests.arl2_harness import OUT_TOL, STATE_TOL, dev, make_pair, out_err, state_err

pytestmark = pytest.mark.gpu

W = Workload("protocol", batch=2, heads=3, head_dim=128, tokens=300, frames=3, denoise_steps=2, seed=21)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _frame_tensors(w, f, p):
    return tuple(dev(x, torch.bfloat16) for x in make_pass_inputs(w, f, p))


def _gates(w, f):
    beta, alpha = make_gates(w, f)
    return dev(beta, torch.float32), dev(alpha, torch.float32)


def _layer(w):
    return Arl2Layer(*[dev(p, torch.bfloat16) for p in make_phi(w)], batch=w.batch, tokens=w.tokens)


def _run(layer, w, frames, stream=None, alt_stream=None):
    """Run frames; returns the outputs of every pass and the state after every frame.  All
    inputs and outputs are created (and synchronised) up front, so that alternating the
    layer between two streams only depends on the library's own stream ordering."""
    inputs = [[(_frame_tensors(w, f, p), _gates(w, f)) for p in range(w.denoise_steps + 1)] for f in range(frames)]
    outs = [layer.new_output() for _ in range(frames * (w.denoise_steps + 1))]
    states = [torch.empty(layer.state_shape, dtype=torch.float32, device="cuda") for _ in range(frames)]
    torch.cuda.synchronize()
    n = 0
    for f in range(frames):
        for p in range(w.denoise_steps + 1):
            s = alt_stream if (alt_stream is not None and (f + p) % 2) else stream
            (q, k, v), (beta, alpha) = inputs[f][p]
            if p < w.denoise_steps:
                layer.denoise_step(q, k, v, out=outs[n], stream=s)
            else:
                layer.commit_frame(q, k, v, beta, alpha, out=outs[n], stream=s)
            n += 1
        st = layer.state(stream=stream)
        torch.cuda.synchronize()
        states[f].copy_(st)
    torch.cuda.synchronize()
    return outs, states


def test_denoise_steps_never_write_state():
    layer = _layer(W)
    _run(layer, W, 2)
    before = layer.state()
    for p in range(5):
        layer.denoise_step(*_frame_tensors(W, 9, p))
    after = layer.state()
    torch.cuda.synchronize()
    assert torch.equal(before, after) and layer.frame_index == 2
    layer.close()


def test_alpha_one_beta_zero_leaves_state_bitwise():
    layer = _layer(W)
    _run(layer, W, 2)
    before = layer.state()
    q, k, v = _frame_tensors(W, 5, 0)
    zeros = torch.zeros((W.batch, W.tokens, W.heads), dtype=torch.float32, device="cuda")
    ones = torch.ones((W.batch, W.heads), dtype=torch.float32, device="cuda")
    layer.commit_frame(q, k, v, zeros, ones, want_output=False)
    after = layer.state()
    torch.cuda.synchronize()
    assert torch.equal(before, after) and layer.frame_index == 3
    layer.close()


def test_runs_are_bitwise_reproducible():
    a_out, a_st = _run(_layer(W), W, 3)
    b_out, b_st = _run(_layer(W), W, 3)
    assert all(torch.equal(x, y) for x, y in zip(a_out, b_out))
    assert all(torch.equal(x, y) for x, y in zip(a_st, b_st))


def test_two_streams_match_one_stream():
    ref_out, ref_st = _run(_layer(W), W, 3)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    out, st = _run(_layer(W), W, 3, stream=s1, alt_stream=s2)
    assert all(torch.equal(x, y) for x, y in zip(ref_out, out))
    assert all(torch.equal(x, y) for x, y in zip(ref_st, st))


def test_checkpoint_and_resume_bitwise():
    full = _layer(W)
    full_out, full_st = _run(full, W, 3)
    first = _layer(W)
    _run(first, W, 1)
    snap, idx = first.state(), first.frame_index
    first.close()
    resumed = _layer(W)
    resumed.load_state(snap, idx)
    assert resumed.frame_index == 1
    outs = []
    for f in (1, 2):
        for p in range(W.denoise_steps + 1):
            q, k, v = _frame_tensors(W, f, p)
            outs.append(resumed.denoise_step(q, k, v) if p < W.denoise_steps
                        else resumed.commit_frame(q, k, v, *_gates(W, f)))
    st = resumed.state()
    torch.cuda.synchronize()
    per = W.denoise_steps + 1
    assert all(torch.equal(x, y) for x, y in zip(full_out[per:], outs))
    assert torch.equal(full_st[-1], st)


def test_every_token_reads_the_same_state():
    """Duplicated query tokens (anywhere in the frame, across query tiles) give bitwise
    identical outputs, and the clean pass's output equals a denoising pass's on the same
    inputs (both read S_{N-1}; the write happens after)."""
    layer = _layer(W)
    _run(layer, W, 1)
    q, k, v = _frame_tensors(W, 1, 0)
    for t in (5, 130, 257, 299):
        q[:, t] = q[:, 3]
    o_den = layer.denoise_step(q, k, v)
    o_clean = layer.commit_frame(q, k, v, *_gates(W, 1))
    torch.cuda.synchronize()
    for t in (5, 130, 257, 299):
        assert torch.equal(o_den[:, t], o_den[:, 3])
    assert torch.equal(o_den, o_clean)
    layer.close()


def test_token_permutation():
    layer, orc = make_pair(W)
    _run(layer, W, 1)
    layer2 = _layer(W)
    _run(layer2, W, 1)
    q, k, v = make_pass_inputs(W, 1, W.denoise_steps)
    beta, alpha = make_gates(W, 1)
    perm = np.random.default_rng(3).permutation(W.tokens)
    o1 = layer.commit_frame(*(dev(x, torch.bfloat16) for x in (q, k, v)), dev(beta, torch.float32),
                            dev(alpha, torch.float32))
    o2 = layer2.commit_frame(*(dev(x[:, perm], torch.bfloat16) for x in (q, k, v)),
                             dev(beta[:, perm], torch.float32), dev(alpha, torch.float32))
    s1, s2 = layer.state().double().cpu().numpy(), layer2.state().double().cpu().numpy()
    o1, o2 = o1.double().cpu().numpy(), o2.double().cpu().numpy()
    # Reordering changes which keys share a 32-key unit, hence the running max that fp16 P is
    # rounded against: differences at the 1e-4 level are rounding; a token-sequential write
    # would differ at order 1.
    e_out, e_state = out_err(o2, o1[:, perm]), state_err(s2, s1)
    assert e_out <= 2e-3, e_out
    assert e_state <= 1e-4, e_state


def test_device_memory_is_constant():
    layer = _layer(W)
    bytes0 = layer.device_bytes
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    _run(layer, W, 3)
    torch.cuda.synchronize()
    assert layer.device_bytes == bytes0
    # the layer allocates nothing after create (torch's cache may hold the test's tensors)
    assert torch.cuda.mem_get_info()[0] >= free0 - 64 * 2**20
    layer.close()


def test_bad_arguments_leave_layer_usable():
    layer = _layer(W)
    q, k, v = _frame_tensors(W, 0, 0)
    with pytest.raises(ValueError):
        layer.denoise_step(q[:, :-1], k, v)
    raw = torch.empty(W.batch * W.tokens * W.heads * W.head_dim + 8, dtype=torch.bfloat16, device="cuda")
    misaligned = raw[4:4 + q.numel()].view(q.shape)
    with pytest.raises(Arl2Error) as ei:
        layer.denoise_step(misaligned, k, v)
    assert ei.value.status == 1
    out = layer.denoise_step(q, k, v)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    layer.close()
    with pytest.raises(Arl2Error):
        layer.denoise_step(q, k, v)


def test_graph_replays_match_eager():
    """Frames captured in HIP graphs (one per input slot, including the state read) and
    replayed repeatedly, with eager work and synchronisation between replays, give bitwise
    the eager results of the same frames."""
    frames = 6
    ref_out, ref_st = _run(_layer(W), W, frames)
    per = W.denoise_steps + 1
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        layer = _layer(W)
        slots = [[(_frame_tensors(W, f, p), _gates(W, f)) for p in range(per)] for f in range(frames)]
        out = layer.new_output()
        st = torch.empty(layer.state_shape, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        graphs = []
        for f in range(frames):  # one graph per frame: inputs differ per frame
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for p in range(per):
                    (q, k, v), (beta, alpha) = slots[f][p]
                    if p < W.denoise_steps:
                        layer.denoise_step(q, k, v, out=out, stream=stream)
                    else:
                        layer.commit_frame(q, k, v, beta, alpha, out=out, stream=stream)
                layer.state(out=st, stream=stream)
            graphs.append(g)
        torch.cuda.synchronize()
        for rep in range(2):  # replay the whole stream twice from S_0
            layer.load_state(torch.zeros_like(st), 0, stream=stream)
            for f in range(frames):
                graphs[f].replay()
                torch.cuda.synchronize()
                scratch = (out.float().sum() + st.sum()).item()  # eager work between replays
                assert scratch == scratch
                assert torch.equal(out, ref_out[(f + 1) * per - 1]), (rep, f)
                assert torch.equal(st, ref_st[f]), (rep, f)
        layer.close()


def test_one_frame_graph_replayed_frame_after_frame():
    """One frame captured once (its denoising passes, the clean pass and the state read, on fixed
    input buffers) and replayed for every frame of a stream, the buffers refilled eagerly between
    replays: each replay advances the state exactly as the eager calls do (an odd number of
    commits per graph, and the same graph every frame)."""
    frames = 5
    ref_out, ref_st = _run(_layer(W), W, frames)
    per = W.denoise_steps + 1
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        layer = _layer(W)
        slots = [(tuple(torch.empty_like(x) for x in _frame_tensors(W, 0, p)),
                  tuple(torch.empty_like(x) for x in _gates(W, 0))) for p in range(per)]
        out = layer.new_output()
        st = torch.empty(layer.state_shape, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for p in range(per):
                (q, k, v), (beta, alpha) = slots[p]
                if p < W.denoise_steps:
                    layer.denoise_step(q, k, v, out=out, stream=stream)
                else:
                    layer.commit_frame(q, k, v, beta, alpha, out=out, stream=stream)
            layer.state(out=st, stream=stream)
        torch.cuda.synchronize()
        layer.load_state(torch.zeros_like(st), 0, stream=stream)
        for f in range(frames):
            for p in range(per):
                for dst, src in zip(slots[p][0] + slots[p][1], _frame_tensors(W, f, p) + _gates(W, f)):
                    dst.copy_(src)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out[(f + 1) * per - 1]), f
            assert torch.equal(st, ref_st[f]), f
        layer.close()
