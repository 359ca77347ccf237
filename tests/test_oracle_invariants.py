"""Pins of the oracle to closed forms, invariants and library routines.

Each test names the statement of "Attend Locally, Remember Linearly" (gist.science technical
summary, sections 2.1 and 2.2; authors' abstract) it pins, and each is chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign, a transposed operand, alpha in
the wrong place, per-token instead of per-frame state access) fails it.
"""
import numpy as np
import pytest
import torch

from oracle import Arl2Oracle, unit_rows
from synth import WORKLOADS, make_gates, make_pass_inputs, make_phi

RNG = np.random.default_rng(1234)


def _rand(*shape):
    return RNG.standard_normal(shape)


def _layer(d=8, heads=2, batch=2, phi_scale=0.3, **kw):
    phis = [np.eye(d)[None] + phi_scale * _rand(heads, d, d) for _ in range(3)]
    return Arl2Oracle(*phis, batch=batch, **kw), phis


def _warm(orc, tokens=6, frames=2):
    """Advance a layer by a few frames of random data so that its state is non-zero."""
    B, H, d = orc.batch, orc.heads, orc.head_dim
    for _ in range(frames):
        q, k, v = (_rand(B, tokens, H, d) for _ in range(3))
        orc.commit(q, k, v, RNG.uniform(0.1, 0.9, (B, tokens, H)), RNG.uniform(0.5, 1.0, (B, H)))
    assert np.abs(orc.state).max() > 1e-3


def _sdpa(q, k, v):
    """Library softmax attention (torch CPU, fp64) per (b, h); q, k, v [B, T, H, d]."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    return o.numpy().transpose(0, 2, 1, 3)


# --- clean-pass updates and the update form (state update, section 2.1; section 2.2) --------

def test_alpha_one_beta_zero_leaves_state_bitwise():
    orc, _ = _layer()
    _warm(orc)
    before = orc.state.copy()
    B, H, d = orc.batch, orc.heads, orc.head_dim
    q, k, v = (_rand(B, 7, H, d) for _ in range(3))
    orc.commit(q, k, v, np.zeros((B, 7, H)), np.ones((B, H)))
    assert np.array_equal(orc.state, before)
    assert orc.frame == 3


def test_denoise_steps_never_write_state():
    orc, _ = _layer()
    _warm(orc)
    before, frame = orc.state.copy(), orc.frame
    for _ in range(5):
        orc.denoise_step(*(_rand(orc.batch, 9, orc.heads, orc.head_dim) for _ in range(3)))
    assert np.array_equal(orc.state, before) and orc.frame == frame


# --- frame-level access (section 2.2; abstract) --------------------------------------------

def test_every_token_reads_the_same_pre_update_state():
    orc, phis = _layer(d=6, heads=1, batch=1)
    _warm(orc)
    s_prev = orc.state[0, 0].copy()
    q, k, v = (_rand(1, 10, 1, 6) for _ in range(3))
    out = orc.commit(q, k, v, RNG.uniform(0.1, 0.9, (1, 10, 1)), np.array([[0.8]]))
    s_new = orc.state[0, 0]
    o_intra = _sdpa(q, k, v)[0, :, 0]
    qp = q[0, :, 0] @ phis[0][0]
    inter = out[0, :, 0] - o_intra
    for t in range(10):
        np.testing.assert_allclose(inter[t], qp[t] @ s_prev, rtol=1e-12, atol=1e-12)
        assert np.abs(inter[t] - qp[t] @ s_new).max() > 1e-6  # the clean pass must not see S_N


def test_token_permutation_equivariance_and_duplicates():
    orc, _ = _layer(d=8, heads=2, batch=1)
    _warm(orc)
    orc2 = Arl2Oracle(orc.phi_q, orc.phi_k, orc.phi_v, batch=1)
    orc2.state = orc.state.copy()
    T = 12
    q, k, v = (_rand(1, T, 2, 8) for _ in range(3))
    q[:, 5] = q[:, 2]  # a duplicated query token
    beta, alpha = RNG.uniform(0.1, 0.9, (1, T, 2)), RNG.uniform(0.5, 1, (1, 2))
    perm = RNG.permutation(T)
    o1 = orc.commit(q, k, v, beta, alpha)
    o2 = orc2.commit(q[:, perm], k[:, perm], v[:, perm], beta[:, perm], alpha)
    np.testing.assert_allclose(o2, o1[:, perm], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(orc2.state, orc.state, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(o1[:, 5], o1[:, 2])


def _token_sequential_state(orc, k, v, beta, alpha):
    """The ablated token-level access: one delta step per token, in token order (one head)."""
    s = orc.state[0, 0].copy()
    kp = unit_rows(k[0, :, 0] @ orc.phi_k[0])
    vp = v[0, :, 0] @ orc.phi_v[0]
    for t in range(len(kp)):
        s = s + beta[0, t, 0] * np.outer(kp[t], vp[t] - kp[t] @ s)
    return alpha[0, 0] * s


def test_permutation_pin_separates_frame_level_from_token_level_access():
    """The permutation pin above would fail for the sequential (token-level) variant, so it
    really pins the frame-level reading."""
    orc, _ = _layer(d=4, heads=1, batch=1)
    _warm(orc)
    T = 10
    k, v = _rand(1, T, 1, 4), _rand(1, T, 1, 4)
    beta, alpha = RNG.uniform(0.3, 0.9, (1, T, 1)), np.array([[0.9]])
    perm = RNG.permutation(T)
    s_a = _token_sequential_state(orc, k, v, beta, alpha)
    s_b = _token_sequential_state(orc, k[:, perm], v[:, perm], beta[:, perm], alpha)
    assert np.abs(s_a - s_b).max() > 1e-6


# --- the intra-frame branch (section 2.1) against a library routine -------------------------

def test_first_frame_is_textbook_attention():
    orc, _ = _layer(d=16, heads=3, batch=2)
    q, k, v = (_rand(2, 20, 3, 16) for _ in range(3))
    np.testing.assert_allclose(orc.denoise_step(q, k, v), _sdpa(q, k, v), rtol=1e-12, atol=1e-13)


def test_zero_query_map_gives_textbook_attention_at_any_state():
    orc, _ = _layer(d=8, heads=2, batch=1)
    _warm(orc)
    orc.phi_q = np.zeros_like(orc.phi_q)
    q, k, v = (_rand(1, 11, 2, 8) for _ in range(3))
    np.testing.assert_allclose(orc.query(q, k, v), _sdpa(q, k, v), rtol=1e-12, atol=1e-13)


def test_equal_keys_single_token_and_linearity_in_v():
    orc, _ = _layer(d=4, heads=1, batch=1)
    q, v = _rand(1, 9, 1, 4), _rand(1, 9, 1, 4)
    k = np.repeat(_rand(1, 1, 1, 4), 9, axis=1)
    np.testing.assert_allclose(orc.query(q, k, v)[0, :, 0], np.repeat(v[0, :, 0].mean(0, keepdims=True), 9, 0),
                               rtol=1e-12, atol=1e-13)
    q1, k1, v1 = (_rand(1, 1, 1, 4) for _ in range(3))
    np.testing.assert_allclose(orc.query(q1, k1, v1), v1, rtol=0, atol=1e-15)
    k = _rand(1, 9, 1, 4)
    v2 = _rand(1, 9, 1, 4)
    np.testing.assert_allclose(orc.query(q, k, v + 3.0 * v2), orc.query(q, k, v) + 3.0 * orc.query(q, k, v2),
                               rtol=1e-12, atol=1e-12)


# --- the delta-rule write (section 2.1, state update) against closed forms -----------------

@pytest.mark.parametrize("alpha", [0.0, 0.37, 1.0])
def test_orthonormal_key_retrieval(alpha):
    """T <= d, phi_k = I, orthonormal key rows: K' S_N = alpha K' S_{N-1} + diag(beta)(V' - K' S_{N-1}).
    At alpha = 1, beta = 1 this is exact delta-rule retrieval K' S_N = V'."""
    d, T = 8, 5
    orc, _ = _layer(d=d, heads=1, batch=1)
    orc.phi_k = np.eye(d)[None]
    _warm(orc)
    s_prev = orc.state[0, 0].copy()
    kq, _ = np.linalg.qr(_rand(d, d))
    k = (3.0 * kq[:T])[None, :, None, :]       # orthogonal rows of norm 3, normalised to 1 by the layer
    v = _rand(1, T, 1, d)
    beta = RNG.uniform(0.1, 1.0, (1, T, 1))
    orc.commit(_rand(1, T, 1, d), k, v, beta, np.array([[alpha]]))
    kp, vp = kq[:T], v[0, :, 0] @ orc.phi_v[0]
    lhs = kp @ orc.state[0, 0]
    rhs = alpha * kp @ s_prev + beta[0, :, 0][:, None] * (vp - kp @ s_prev)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-11)
    if alpha == 1.0:
        orc2 = Arl2Oracle(orc.phi_q, orc.phi_k, orc.phi_v, batch=1)
        orc2.state = orc.state.copy()
        orc2.commit(_rand(1, T, 1, d), k, v, np.ones((1, T, 1)), np.array([[1.0]]))
        np.testing.assert_allclose(kp @ orc2.state[0, 0], vp, rtol=1e-11, atol=1e-11)


def test_square_orthogonal_keys_overwrite_history():
    """T = d orthogonal keys, alpha = beta = 1: S_N = K'^T V' whatever S_{N-1} was."""
    d = 6
    orc, _ = _layer(d=d, heads=1, batch=1)
    orc.phi_k = np.eye(d)[None]
    _warm(orc)
    kq, _ = np.linalg.qr(_rand(d, d))
    v = _rand(1, d, 1, d)
    orc.commit(_rand(1, d, 1, d), (0.5 * kq)[None, :, None, :], v, np.ones((1, d, 1)), np.ones((1, 1)))
    np.testing.assert_allclose(orc.state[0, 0], kq.T @ (v[0, :, 0] @ orc.phi_v[0]), rtol=1e-11, atol=1e-11)


def test_affine_form_of_the_write():
    """S_N = (alpha I - K'^T diag(beta) K') S_{N-1} + K'^T diag(beta) V' for general keys."""
    orc, phis = _layer(d=5, heads=1, batch=1)
    _warm(orc)
    s_prev = orc.state[0, 0].copy()
    T = 9
    k, v = _rand(1, T, 1, 5), _rand(1, T, 1, 5)
    beta, alpha = RNG.uniform(0.1, 0.9, (1, T, 1)), 0.6
    orc.commit(_rand(1, T, 1, 5), k, v, beta, np.array([[alpha]]))
    kp = k[0, :, 0] @ phis[1][0]
    kp = kp / np.linalg.norm(kp, axis=1, keepdims=True)
    vp = v[0, :, 0] @ phis[2][0]
    bk = beta[0, :, 0][:, None] * kp
    want = (alpha * np.eye(5) - kp.T @ bk) @ s_prev + bk.T @ vp
    np.testing.assert_allclose(orc.state[0, 0], want, rtol=1e-11, atol=1e-11)


def test_scalar_head_recurrence_closed_form():
    """d = 1: K' = sign(k phi_k), and S_N = (alpha - sum beta) S + sum beta k' v phi_v, iterated."""
    orc = Arl2Oracle(np.full((1, 1, 1), 0.7), np.full((1, 1, 1), -2.0), np.full((1, 1, 1), 1.5), batch=1)
    s = 0.0
    for _ in range(6):
        T = 4
        k, v = _rand(1, T, 1, 1), _rand(1, T, 1, 1)
        beta, alpha = RNG.uniform(0, 0.2, T), RNG.uniform(0.5, 1.0)
        orc.commit(_rand(1, T, 1, 1), k, v, beta[None, :, None], np.array([[alpha]]))
        kp = np.sign(-2.0 * k[0, :, 0, 0])
        s = (alpha - beta.sum()) * s + np.sum(beta * kp * 1.5 * v[0, :, 0, 0])
        np.testing.assert_allclose(orc.state[0, 0, 0, 0], s, rtol=1e-12, atol=1e-14)


# --- the 1x1 feature maps (section 2.1, adaptation): row-vector convention ------------------

def test_identity_maps():
    d = 6
    eye = np.eye(d)[None]
    orc = Arl2Oracle(eye, eye, eye, batch=1)
    s = _rand(d, d)
    orc.state[0, 0] = s
    q, k, v = (_rand(1, 7, 1, d) for _ in range(3))
    np.testing.assert_allclose(orc.query(q, k, v) - _sdpa(q, k, v), (q[0, :, 0] @ s)[None, :, None], rtol=1e-12,
                               atol=1e-12)
    beta = RNG.uniform(0.1, 0.9, (1, 7, 1))
    new = orc.next_state(k, v, beta, np.array([[0.5]]))
    kn = k[0, :, 0] / np.linalg.norm(k[0, :, 0], axis=1, keepdims=True)
    want = 0.5 * s + kn.T @ (beta[0, :, 0][:, None] * (v[0, :, 0] - kn @ s))
    np.testing.assert_allclose(new[0, 0], want, rtol=1e-12, atol=1e-12)


def test_asymmetric_maps_fix_the_convention():
    """phi with a single off-diagonal 1 at [0, 1]: q' = q phi puts q[0] into column 1.  The
    transposed convention would put q[1] into column 0 and fails this test."""
    d = 4
    e01 = np.zeros((1, d, d))
    e01[0, 0, 1] = 1.0
    perm = np.eye(d)[[2, 0, 3, 1]][None]           # a permutation used as phi_k and phi_v
    orc = Arl2Oracle(e01, perm, perm, batch=1)
    s = _rand(d, d)
    orc.state[0, 0] = s
    q, k, v = (_rand(1, 5, 1, d) for _ in range(3))
    inter = (orc.query(q, k, v) - _sdpa(q, k, v))[0, :, 0]
    np.testing.assert_allclose(inter, np.outer(q[0, :, 0, 0], s[1]), rtol=1e-12, atol=1e-12)
    # the write: with S = 0, alpha = 1, S_1 = (K P / ||.||)^T diag(beta) (V P)
    orc.state[0, 0] = 0.0
    beta = RNG.uniform(0.1, 0.9, (1, 5, 1))
    new = orc.next_state(k, v, beta, np.ones((1, 1)))[0, 0]
    kp = k[0, :, 0][:, [1, 3, 0, 2]]                  # (K P)[t, j] = K[t, i] where P[i, j] = 1
    kp = kp / np.linalg.norm(kp, axis=1, keepdims=True)
    vp = v[0, :, 0][:, [1, 3, 0, 2]]
    np.testing.assert_allclose(new, kp.T @ (beta[0, :, 0][:, None] * vp), rtol=1e-12, atol=1e-12)


def test_unit_rows():
    x = _rand(10, 7)
    x[3] = 0.0
    x[4] = 1e-9
    y = unit_rows(x, 1e-6)
    np.testing.assert_allclose(np.linalg.norm(y[[0, 1, 2, 5, 6, 7, 8, 9]], axis=1), 1.0, rtol=1e-14)
    assert np.all(y[3] == 0.0)
    np.testing.assert_allclose(y[4], x[4] / 1e-6, rtol=1e-15)


# --- precision: fp32 oracle mode tracks fp64 over a long stream -----------------------------

def test_fp32_mode_tracks_fp64_over_many_commits():
    w = WORKLOADS["tiny"].with_(tokens=64, frames=60)
    phis = make_phi(w)
    o64 = Arl2Oracle(*phis, batch=1)
    o32 = Arl2Oracle(*phis, batch=1, dtype=np.float32)
    for f in range(w.frames):
        _, k, v = make_pass_inputs(w, f, w.denoise_steps)
        beta, alpha = make_gates(w, f)
        o64.state = o64.next_state(k, v, beta, alpha)
        o32.state = o32.next_state(k, v, beta, alpha)
    rel = np.linalg.norm(o32.state - o64.state) / np.linalg.norm(o64.state)
    assert rel < 1e-5, rel
