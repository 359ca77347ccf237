"""Pins of the backward oracle (CPU only).

The gradients of oracle.bwd_oracle are checked against central finite differences of a loss
computed with the forward oracle alone (oracle.arl2_oracle.Arl2Oracle: query / commit), which is
pinned on its own; every scalar input is perturbed on tiny streams, random directions on larger
ones.  Plus closed forms, the token-permutation symmetry of frame-level access, and planted
mistakes that must each fail a pin.

Source: "Attend Locally, Remember Linearly" technical summary (gist.science), sections 2.1-2.2
(the forward) and 2.3 (end-to-end distillation through the layer, which needs these gradients).
"""
import numpy as np
import pytest

import oracle.bwd_oracle as bo
from oracle import Arl2Oracle


def make_stream(rng, B=1, H=2, d=3, T=4, frames=3, passes=2, none_at=None, small_k=False):
    phi = [np.eye(d)[None].repeat(H, 0) + 0.3 * rng.standard_normal((H, d, d)) for _ in range(3)]
    fr, d_outs = [], []
    for n in range(frames):
        ps = []
        for p in range(passes):
            q, k, v = (rng.standard_normal((B, T, H, d)) for _ in range(3))
            if small_k:
                k[:, ::2] *= 0.05  # rows whose |k phi_k| falls below a large eps
            ps.append((q, k, v))
        fr.append({"passes": ps, "beta": rng.uniform(0.1, 0.9, (B, T, H)), "alpha": rng.uniform(0.3, 0.95, (B, H))})
        d_outs.append([None if (n, p) == none_at else rng.standard_normal((B, T, H, d)) for p in range(passes)])
    g_last = rng.standard_normal((B, H, d, d))
    s0 = 0.5 * rng.standard_normal((B, H, d, d))
    return phi, fr, d_outs, g_last, s0


def loss(phi, frames, d_outs, g_last, s0, eps=1e-6):
    """sum of <dO, out> over every pass with an output gradient, plus <G_F, S_F>: computed with the
    forward oracle only."""
    B = frames[0]["passes"][0][0].shape[0]
    orc = Arl2Oracle(*phi, batch=B, knorm_eps=eps)
    orc.state = np.array(s0, dtype=np.float64)
    total = 0.0
    for n, fr in enumerate(frames):
        last = len(fr["passes"]) - 1
        for p, (q, k, v) in enumerate(fr["passes"]):
            out = orc.query(q, k, v) if p < last else orc.commit(q, k, v, fr["beta"], fr["alpha"])
            if d_outs[n][p] is not None:
                total += float(np.sum(d_outs[n][p] * out))
    return total + float(np.sum(g_last * orc.state))


def leaves(phi, frames, s0):
    """(name, array, gradient key) for every input the loss depends on."""
    out = [(f"phi_{c}", phi[i], ("dphi_" + c,)) for i, c in enumerate("qkv")]
    out.append(("s0", s0, ("ds0",)))
    for n, fr in enumerate(frames):
        for p, qkv in enumerate(fr["passes"]):
            for i, c in enumerate("qkv"):
                out.append((f"{c}[{n}][{p}]", qkv[i], ("d" + c, n, p)))
        out.append((f"beta[{n}]", fr["beta"], ("dbeta", n)))
        out.append((f"alpha[{n}]", fr["alpha"], ("dalpha", n)))
    return out


def grad_of(res, key):
    g = res[key[0]]
    for i in key[1:]:
        g = g[i]
    return g


def backward(phi, frames, d_outs, g_last, s0, eps=1e-6):
    return bo.layer_backward(*phi, frames, d_outs, g_last=g_last, s0=s0, eps=eps)


def check_all_scalars(rng, eps=1e-6, h=1e-6, **kw):
    phi, fr, d_outs, g_last, s0 = make_stream(rng, **kw)
    res = backward(phi, fr, d_outs, g_last, s0, eps)
    worst = 0.0
    for name, arr, key in leaves(phi, fr, s0):
        g = np.asarray(grad_of(res, key))
        fd = np.empty(arr.shape)
        for idx in np.ndindex(arr.shape):
            x0 = arr[idx]
            arr[idx] = x0 + h
            lp = loss(phi, fr, d_outs, g_last, s0, eps)
            arr[idx] = x0 - h
            lm = loss(phi, fr, d_outs, g_last, s0, eps)
            arr[idx] = x0
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(g - fd).max() / max(1.0, np.abs(fd).max())
        assert err < 1e-6, (name, err)
        worst = max(worst, err)
    return worst


def test_finite_differences_every_scalar():
    check_all_scalars(np.random.default_rng(1))


def test_finite_differences_two_streams_and_a_pass_without_gradient():
    check_all_scalars(np.random.default_rng(2), B=2, H=1, d=2, T=3, frames=2, passes=3, none_at=(1, 0))


def test_finite_differences_key_norm_below_eps():
    """Rows of K phi_k shorter than eps take the constant branch of max(|u|, eps)."""
    check_all_scalars(np.random.default_rng(3), eps=0.5, small_k=True)


def test_directional_derivatives_larger_stream():
    """T = 37, d = 8, 3 frames of 3 passes: <grad, delta> against the central difference along
    random directions over all inputs at once."""
    rng = np.random.default_rng(4)
    phi, fr, d_outs, g_last, s0 = make_stream(rng, B=1, H=2, d=8, T=37, frames=3, passes=3)
    res = backward(phi, fr, d_outs, g_last, s0)
    lv = leaves(phi, fr, s0)
    for _ in range(4):
        dirs = [rng.standard_normal(a.shape) for _, a, _ in lv]
        pred = sum(float(np.sum(np.asarray(grad_of(res, key)) * dd)) for (_, _, key), dd in zip(lv, dirs))
        h = 1e-5
        vals = []
        for sgn in (1, -1):
            for (_, a, _), dd in zip(lv, dirs):
                a += sgn * h * dd
            vals.append(loss(phi, fr, d_outs, g_last, s0))
            for (_, a, _), dd in zip(lv, dirs):
                a -= sgn * h * dd
        fd = (vals[0] - vals[1]) / (2 * h)
        assert abs(pred - fd) < 1e-6 * max(1.0, abs(fd)), (pred, fd)


def test_single_token_pass_closed_form():
    """T = 1 and S_{N-1} = 0: the softmax weight is 1, so dV = dO and dQ = dK = 0."""
    rng = np.random.default_rng(5)
    q, k, v, d_o = (rng.standard_normal((1, 1, 2, 4)) for _ in range(4))
    dq, dk, dv, ds, dphi = bo.pass_backward(q, k, v, d_o, np.zeros((1, 2, 4, 4)), rng.standard_normal((2, 4, 4)), 0.5)
    np.testing.assert_array_equal(dq, 0.0)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_array_equal(dv, d_o)
    np.testing.assert_array_equal(dphi, 0.0)


def test_identity_write_passes_the_state_gradient_through():
    """beta = 0 and alpha = 1 make S_N = S_{N-1}: dS_{N-1} = G, no K or V gradient, dalpha = <G, S>."""
    rng = np.random.default_rng(6)
    B, T, H, d = 1, 5, 2, 4
    k, v = rng.standard_normal((B, T, H, d)), rng.standard_normal((B, T, H, d))
    s, g = rng.standard_normal((B, H, d, d)), rng.standard_normal((B, H, d, d))
    phi = rng.standard_normal((H, d, d))
    dk, dv, dbeta, dalpha, ds, dpk, dpv = bo.write_backward(k, v, np.zeros((B, T, H)), np.ones((B, H)), s, g, phi, phi)
    np.testing.assert_array_equal(ds, g)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_array_equal(dv, 0.0)
    np.testing.assert_allclose(dalpha, np.einsum("bhij,bhij->bh", g, s), rtol=1e-14)


def test_token_permutation_symmetry():
    """Frame-level access: permuting the tokens of every frame permutes the token gradients and
    leaves the gradients of phi, alpha and S_0 unchanged."""
    rng = np.random.default_rng(7)
    phi, fr, d_outs, g_last, s0 = make_stream(rng, B=1, H=2, d=4, T=6, frames=2, passes=2)
    res = backward(phi, fr, d_outs, g_last, s0)
    perm = rng.permutation(6)
    fr_p = [{"passes": [tuple(x[:, perm] for x in qkv) for qkv in f["passes"]], "beta": f["beta"][:, perm],
             "alpha": f["alpha"]} for f in fr]
    d_p = [[x[:, perm] for x in row] for row in d_outs]
    res_p = backward(phi, fr_p, d_p, g_last, s0)
    for key in ("dphi_q", "dphi_k", "dphi_v", "ds0"):
        np.testing.assert_allclose(res_p[key], res[key], rtol=1e-12, atol=1e-12)
    for n in range(2):
        np.testing.assert_allclose(res_p["dalpha"][n], res["dalpha"][n], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res_p["dbeta"][n], res["dbeta"][n][:, perm], rtol=1e-12, atol=1e-12)
        for c in ("dq", "dk", "dv"):
            for p in range(2):
                np.testing.assert_allclose(res_p[c][n][p], res[c][n][p][:, perm], rtol=1e-12, atol=1e-12)


# --- planted mistakes: each must fail a finite-difference pin --------------------------------------
_ORIG = {n: getattr(bo, n) for n in ("softmax_attention_bwd", "inter_read_bwd", "unit_rows_bwd", "delta_write_bwd")}


def _no_rowsum(q, k, v, d_o, scale):
    a = (q @ k.T) * scale
    p = np.exp(a - a.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    da = p * (d_o @ v.T)
    return scale * (da @ k), scale * (da.T @ q), p.T @ d_o


def _read_ds_transposed(q, d_o, s_prev, phi_q):
    a, b, c = _ORIG["inter_read_bwd"](q, d_o, s_prev, phi_q)
    return a, b, c.T


def _no_norm_projection(x, dy, eps=1e-6):
    n = np.sqrt(np.sum(x * x, axis=1, keepdims=True))
    return dy / np.maximum(n, eps)


def _no_residual_term(s_prev, k_prime, v_prime, beta, alpha, g):
    ds, dkp, dvp, dbeta, dalpha = _ORIG["delta_write_bwd"](s_prev, k_prime, v_prime, beta, alpha, g)
    return ds, dkp + (beta[:, None] * (k_prime @ g)) @ s_prev.T, dvp, dbeta, dalpha


def _no_decay_term(s_prev, k_prime, v_prime, beta, alpha, g):
    ds, dkp, dvp, dbeta, dalpha = _ORIG["delta_write_bwd"](s_prev, k_prime, v_prime, beta, alpha, g)
    return ds - alpha * g, dkp, dvp, dbeta, dalpha


MUTANTS = {"softmax without the rowsum term": ("softmax_attention_bwd", _no_rowsum),
           "inter-read state gradient transposed": ("inter_read_bwd", _read_ds_transposed),
           "key normalisation without its projection": ("unit_rows_bwd", _no_norm_projection),
           "dK' without the residual's -dR S^T term": ("delta_write_bwd", _no_residual_term),
           "dS without the decay term": ("delta_write_bwd", _no_decay_term)}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    fn, mutant = MUTANTS[name]
    monkeypatch.setattr(bo, fn, mutant)
    with pytest.raises(AssertionError):
        check_all_scalars(np.random.default_rng(1))
