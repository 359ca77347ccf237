"""GPU parity of the layer's backward (include/arl2_bwd.h) against the backward oracle
(oracle.bwd_oracle.layer_backward), frames walked in reverse.

Bars (derived from the arithmetic of each path):
  dq, dk, dv      max |err| / rms(oracle) <= 2e-2: the softmax branch's backward multiplies fp16
                  operands (P, dS and dO rounded at relative step 2^-11) with fp32 accumulation,
                  and its scores recompute the forward's bf16 Q K^T; the forward output's bar;
  dbeta           max |err| / rms(oracle) <= 1e-3;
  dalpha, dS_0, dphi_q, dphi_k, dphi_v   ||err||_F / ||oracle||_F <= 1e-3 (split-bf16 products,
                  about fp32 accuracy, as the forward's state bar).
Inputs: the seeded synthetic streams (synth/), output gradients ~ N(0, 1), dL/dS after the last
frame ~ N(0, 1/d).  The forward states S_{N-1} fed to the GPU are the oracle's, in fp32.
"""
import numpy as np
import pytest
import torch

from gated_delta_linear_amd import Arl2Backward
from oracle import layer_backward
from oracle.bwd_oracle import forward_states
from synth import (WORKLOADS, Workload, make_gates, make_out_grad, make_pass_inputs, make_phi, make_state_grad,
                   round_bf16)
from tests.arl2_harness import dev, log, out_err, state_err

pytestmark = pytest.mark.gpu

TOK_TOL = 2e-2
PRECISE_TOL = 1e-3


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def make_stream(w, frames, passes, no_grad=(), k_scale_rows=None):
    """Frames of w with `passes` passes each (the last is the clean pass); (frame, pass) pairs in
    no_grad get no output gradient.  k_scale_rows: (scale, every) multiplies every `every`-th
    token row of K by scale (keys whose mapped norm falls below knorm_eps)."""
    fr, d_outs = [], []
    for n in range(frames):
        ps = []
        for p in range(passes):
            q, k, v = make_pass_inputs(w, n, p)
            if k_scale_rows:
                k = k.copy()
                k[:, ::k_scale_rows[1]] *= np.float32(k_scale_rows[0])  # exact in bf16 for powers of 2
            ps.append((q, k, v))
        beta, alpha = make_gates(w, n)
        fr.append({"passes": ps, "beta": beta, "alpha": alpha})
        d_outs.append([None if (n, p) in no_grad else make_out_grad(w, n, p) for p in range(passes)])
    return fr, d_outs


def gpu_backward(w, phis, frames, d_outs, g_last, knorm_eps=0.0):
    """The sweep through libarl2; returns the same dict layout as layer_backward (numpy)."""
    eps = knorm_eps if knorm_eps > 0 else 1e-6
    states = forward_states(phis[1].astype(np.float64), phis[2].astype(np.float64), frames,
                            np.zeros((w.batch, w.heads, w.head_dim, w.head_dim)), eps)
    bw = Arl2Backward(*[dev(p, torch.bfloat16) for p in phis], batch=w.batch, tokens=w.tokens, knorm_eps=knorm_eps)
    bw.begin(dev(g_last, torch.float32))
    F, P = len(frames), len(frames[0]["passes"])
    res = {key: [None] * F for key in ("dq", "dk", "dv", "dbeta", "dalpha")}
    for n in range(F - 1, -1, -1):
        s_prev = dev(states[n], torch.float32)
        fr = frames[n]
        dq_n, dk_n, dv_n = [], [], []
        for p, (q, k, v) in enumerate(fr["passes"]):
            if d_outs[n][p] is None:
                z = torch.zeros(bw.frame_shape, dtype=torch.float32, device="cuda")
                dq_n.append(z), dk_n.append(z.clone()), dv_n.append(z.clone())
                continue
            g = bw.pass_(*(dev(x, torch.bfloat16) for x in (q, k, v)), s_prev, dev(d_outs[n][p], torch.float32))
            dq_n.append(g[0]), dk_n.append(g[1]), dv_n.append(g[2])
        _, k, v = fr["passes"][-1]
        dbeta, dalpha = bw.commit(dev(k, torch.bfloat16), dev(v, torch.bfloat16), dev(fr["beta"], torch.float32),
                                  dev(fr["alpha"], torch.float32), s_prev, dk_n[-1], dv_n[-1])
        res["dq"][n] = [x.cpu().numpy() for x in dq_n]
        res["dk"][n] = [x.cpu().numpy() for x in dk_n]
        res["dv"][n] = [x.cpu().numpy() for x in dv_n]
        res["dbeta"][n] = dbeta.cpu().numpy()
        res["dalpha"][n] = dalpha.cpu().numpy()
    ds0, dpq, dpk, dpv = bw.read()
    torch.cuda.synchronize()
    res.update(ds0=ds0.cpu().numpy(), dphi_q=dpq.cpu().numpy(), dphi_k=dpk.cpu().numpy(), dphi_v=dpv.cpu().numpy())
    bw.close()
    return res


def compare(got, want, d_outs, heads=None):
    """Largest errors of each kind; heads: the head indices the oracle ran on (all if None)."""
    sel = (lambda x, ax: x) if heads is None else (lambda x, ax: np.take(x, heads, axis=ax))
    tok = prec = 0.0
    for n in range(len(want["dq"])):
        for p in range(len(want["dq"][n])):
            if d_outs[n][p] is None and p < len(want["dq"][n]) - 1:
                continue
            for key in ("dq", "dk", "dv"):
                w_ = want[key][n][p]
                if not np.any(w_):
                    continue
                tok = max(tok, out_err(sel(got[key][n][p], 2), w_))
        prec = max(prec, out_err(sel(got["dbeta"][n], 2), want["dbeta"][n]),
                   state_err(sel(got["dalpha"][n], 1), want["dalpha"][n]))
    prec = max(prec, state_err(sel(got["ds0"], 1), want["ds0"]),
               *(state_err(sel(got[key], 0), want[key]) for key in ("dphi_q", "dphi_k", "dphi_v")))
    return tok, prec


def run_case(w, frames, passes, no_grad=(), knorm_eps=0.0, k_scale_rows=None):
    phis = make_phi(w)
    fr, d_outs = make_stream(w, frames, passes, no_grad, k_scale_rows)
    g_last = make_state_grad(w)
    log(f"bwd {w.name}: B{w.batch} H{w.heads} d{w.head_dim} T{w.tokens} frames {frames} passes {passes}")
    got = gpu_backward(w, phis, fr, d_outs, g_last, knorm_eps)
    want = layer_backward(*(p.astype(np.float64) for p in phis), fr, d_outs, g_last=g_last,
                          eps=knorm_eps if knorm_eps > 0 else 1e-6)
    tok, prec = compare(got, want, d_outs)
    log(f"  token grads {tok:.3e}, state / map / gate grads {prec:.3e}")
    return tok, prec


SMALL = [  # (batch, heads, d, T, frames, passes)
    (1, 1, 64, 1, 2, 2),
    (1, 2, 64, 37, 3, 2),
    (2, 2, 64, 200, 2, 3),
    (1, 2, 128, 64, 2, 2),
    (1, 2, 128, 100, 2, 2),  # two 64-row blocks: the staging loops' tail without a third block
    (1, 1, 64, 128, 2, 2),   # two full blocks
    (1, 1, 128, 129, 3, 2),
    (2, 3, 128, 200, 2, 2),
    (1, 2, 128, 333, 2, 2),
]


@pytest.mark.parametrize("B,H,d,T,frames,passes", SMALL)
def test_small_shapes(B, H, d, T, frames, passes):
    w = Workload(f"bwd_{B}_{H}_{d}_{T}", batch=B, heads=H, head_dim=d, tokens=T, frames=frames,
                 denoise_steps=passes - 1, seed=500 + T + d)
    tok, prec = run_case(w, frames, passes)
    assert tok <= TOK_TOL and prec <= PRECISE_TOL, (tok, prec)


def test_passes_without_output_gradient():
    """A denoising pass outside the loss, and a frame whose clean pass has no output gradient (its
    dk, dv come from the state write alone)."""
    w = Workload("bwd_nograd", batch=1, heads=2, head_dim=128, tokens=150, frames=3, denoise_steps=2, seed=61)
    tok, prec = run_case(w, 3, 3, no_grad={(2, 0), (1, 2)})
    assert tok <= TOK_TOL and prec <= PRECISE_TOL, (tok, prec)


def test_key_norm_below_eps():
    """knorm_eps = 4 with every third key scaled by 1/16: those keys' mapped norms (about
    sqrt(d) / 16) take the constant branch of max(|u|, eps)."""
    w = Workload("bwd_eps", batch=1, heads=2, head_dim=64, tokens=96, frames=2, denoise_steps=1, seed=62)
    tok, prec = run_case(w, 2, 2, knorm_eps=4.0, k_scale_rows=(1.0 / 16, 3))
    assert tok <= TOK_TOL and prec <= PRECISE_TOL, (tok, prec)


@pytest.mark.parametrize("d,T", [(128, 100), (64, 257)])
def test_strongly_negative_scores(d, T):
    """Every score far below zero: q = -16 u + noise, k = u + noise with u of +-1 entries per
    head, so scores sit near -16 d (log-sum-exp near -260 in log2 units at d = 128).  At a ragged
    T the keys that pad the last 64-key block score 0, and exp2(score scale log2 e - lse) there
    would be about 2^260, infinite in fp32: the attention backward must keep such keys from
    reaching any gradient.  (The keys' shared part u is kept small: dq sums dS over keys, whose
    exact sum is zero, so a large shared key part would magnify dS's fp16 rounding.)"""
    w = Workload(f"bwd_neg_{d}_{T}", batch=1, heads=2, head_dim=d, tokens=T, frames=2, denoise_steps=1, seed=70 + T)
    rng = np.random.default_rng(71 + T)
    u = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=(1, 1, w.heads, d))
    fr, d_outs = make_stream(w, 2, 2)
    for f in fr:
        f["passes"] = [(round_bf16(-16 * u + 0.5 * q), round_bf16(u + 0.25 * k), v) for q, k, v in f["passes"]]
    phis = make_phi(w)
    g_last = make_state_grad(w)
    got = gpu_backward(w, phis, fr, d_outs, g_last)
    for key in ("dq", "dk", "dv"):
        assert all(np.isfinite(x).all() for row in got[key] for x in row), key
    want = layer_backward(*(p.astype(np.float64) for p in phis), fr, d_outs, g_last=g_last, eps=1e-6)
    tok, prec = compare(got, want, d_outs)
    log(f"bwd negative scores d={d} T={T}: token grads {tok:.3e}, state / map / gate grads {prec:.3e}")
    assert tok <= TOK_TOL and prec <= PRECISE_TOL, (tok, prec)


def test_dit480p_two_frames():
    """The DiT-layer shape (12 heads, d = 128, 1560 tokens), 2 frames of a denoising pass and the
    clean pass; the oracle runs on heads 0, 5 and 11 (heads are independent)."""
    w = WORKLOADS["dit480p"]
    heads = [0, 5, 11]
    phis = make_phi(w)
    fr, d_outs = make_stream(w, 2, 2)
    g_last = make_state_grad(w)
    got = gpu_backward(w, phis, fr, d_outs, g_last)
    sub = [{"passes": [tuple(x[:, :, heads] for x in qkv) for qkv in f["passes"]], "beta": f["beta"][:, :, heads],
            "alpha": f["alpha"][:, heads]} for f in fr]
    d_sub = [[x[:, :, heads] for x in row] for row in d_outs]
    want = layer_backward(*(p[heads].astype(np.float64) for p in phis), sub, d_sub, g_last=g_last[:, heads])
    tok, prec = compare(got, want, d_sub, heads=heads)
    log(f"bwd dit480p (heads {heads}): token grads {tok:.3e}, state / map / gate grads {prec:.3e}")
    assert tok <= TOK_TOL and prec <= PRECISE_TOL, (tok, prec)


def test_backward_is_bitwise_reproducible():
    w = Workload("bwd_repro", batch=2, heads=2, head_dim=128, tokens=257, frames=2, denoise_steps=1, seed=63)
    phis = make_phi(w)
    fr, d_outs = make_stream(w, 2, 2)
    g_last = make_state_grad(w)
    a = gpu_backward(w, phis, fr, d_outs, g_last)
    b = gpu_backward(w, phis, fr, d_outs, g_last)
    for key in ("ds0", "dphi_q", "dphi_k", "dphi_v"):
        assert np.array_equal(a[key], b[key]), key
    for key in ("dq", "dk", "dv"):
        for n in range(2):
            for p in range(2):
                assert np.array_equal(a[key][n][p], b[key][n][p]), (key, n, p)


def test_calls_on_alternating_streams_match_one_stream():
    """Every call of a sweep on a different stream than the one before (the library makes each
    new stream wait for the previous one): gradients bitwise equal to the one-stream sweep."""
    w = Workload("bwd_streams", batch=1, heads=2, head_dim=128, tokens=200, frames=3, denoise_steps=1, seed=64)
    phis = make_phi(w)
    fr, d_outs = make_stream(w, 3, 2)
    g_last = make_state_grad(w)
    states = forward_states(phis[1].astype(np.float64), phis[2].astype(np.float64), fr,
                            np.zeros((w.batch, w.heads, w.head_dim, w.head_dim)))
    staged = [([tuple(dev(x, torch.bfloat16) for x in qkv) for qkv in f["passes"]], dev(f["beta"], torch.float32),
               dev(f["alpha"], torch.float32), dev(states[n], torch.float32)) for n, f in enumerate(fr)]
    d_dev = [[dev(x, torch.float32) for x in row] for row in d_outs]
    g_dev = dev(g_last, torch.float32)
    torch.cuda.synchronize()

    def sweep(streams):
        pick = iter(streams * 64)
        bw = Arl2Backward(*[dev(p, torch.bfloat16) for p in phis], batch=w.batch, tokens=w.tokens)
        bw.begin(g_dev, stream=next(pick))
        got = []
        for n in range(len(fr) - 1, -1, -1):
            passes, beta, alpha, s_prev = staged[n]
            grads = [bw.pass_(*qkv, s_prev, d_dev[n][p], stream=next(pick)) for p, qkv in enumerate(passes)]
            _, k, v = passes[-1]
            db, da = bw.commit(k, v, beta, alpha, s_prev, grads[-1][1], grads[-1][2], stream=next(pick))
            got += [x for g in grads for x in g] + [db, da]
        got += list(bw.read(stream=next(pick)))
        torch.cuda.synchronize()
        bw.close()
        return [x.cpu().numpy() for x in got]

    one = sweep([torch.cuda.current_stream()])
    two = sweep([torch.cuda.Stream(), torch.cuda.Stream()])  # default priority
    assert len(one) == len(two)
    for i, (a, b) in enumerate(zip(one, two)):
        assert np.array_equal(a, b), i
