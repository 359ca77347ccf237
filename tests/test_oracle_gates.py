"""Pins of the gate projections in the oracle (CPU only): scalar brute force, closed forms and
invariants, and planted mistakes that must each fail a pin.

Source: "Attend Locally, Remember Linearly" technical summary (gist.science), section 2.1 (alpha,
the forget gate, and beta, the learning rate, are learned projections of the tokens) and section
4 (experimental results, ablations: head-wise gates); the frame-level write takes one alpha per (stream, head) and frame, so the
per-token alpha logits are averaged over the frame before the sigmoid (the reading taken here).
"""
import math

import numpy as np
import pytest

import oracle.arl2_oracle as ora

RNG = np.random.default_rng(77)


def _inputs(B=2, T=5, H=3, dm=8):
    x = RNG.standard_normal((B, T, dm))
    w = RNG.standard_normal((2 * H, dm)) / math.sqrt(dm)
    b = RNG.standard_normal(2 * H)
    return x, w, b


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def test_brute_force_scalar_loops():
    x, w, b = _inputs()
    beta, alpha = ora.gate_projections(x, w, b, beta_scale=0.3)
    B, T, dm = x.shape
    H = w.shape[0] // 2
    for bb in range(B):
        for h in range(H):
            zs = []
            for t in range(T):
                zb = sum(x[bb, t, i] * w[h, i] for i in range(dm)) + b[h]
                assert abs(beta[bb, t, h] - 0.3 * _sig(zb)) < 1e-12
                zs.append(sum(x[bb, t, i] * w[H + h, i] for i in range(dm)))
            assert abs(alpha[bb, h] - _sig(sum(zs) / T + b[H + h])) < 1e-12


def test_zero_weights_give_the_biases():
    x, w, b = _inputs()
    beta, alpha = ora.gate_projections(x, np.zeros_like(w), b, beta_scale=2.0)
    H = w.shape[0] // 2
    np.testing.assert_allclose(beta, np.broadcast_to(2.0 / (1.0 + np.exp(-b[:H])), beta.shape), rtol=0, atol=1e-15)
    np.testing.assert_allclose(alpha, np.broadcast_to(1.0 / (1.0 + np.exp(-b[H:])), alpha.shape), rtol=0, atol=1e-15)


def test_alpha_is_the_sigmoid_of_the_mean_logit():
    """Two tokens whose alpha logits are 0 and 4 (bias 0): alpha = sigmoid(2), not the mean of
    sigmoid(0) and sigmoid(4)."""
    H, dm = 1, 2
    w = np.array([[1.0, 0.0], [0.0, 1.0]])  # beta row, alpha row
    x = np.array([[[0.0, 0.0], [0.0, 4.0]]])
    _, alpha = ora.gate_projections(x, w, np.zeros(2 * H))
    assert abs(alpha[0, 0] - _sig(2.0)) < 1e-15


def test_token_permutation():
    """Permuting a frame's tokens permutes beta and leaves alpha unchanged."""
    x, w, b = _inputs(T=9)
    perm = RNG.permutation(9)
    beta, alpha = ora.gate_projections(x, w, b)
    beta_p, alpha_p = ora.gate_projections(x[:, perm], w, b)
    np.testing.assert_allclose(beta_p, beta[:, perm], rtol=0, atol=1e-15)
    np.testing.assert_allclose(alpha_p, alpha, rtol=0, atol=1e-14)


def test_head_wise_gates_use_their_own_rows():
    """Changing head 1's weights changes only head 1's gates."""
    x, w, b = _inputs(H=3)
    beta, alpha = ora.gate_projections(x, w, b)
    w2 = w.copy()
    w2[1] += 1.0
    w2[3 + 1] -= 1.0
    beta2, alpha2 = ora.gate_projections(x, w2, b)
    keep = [0, 2]
    np.testing.assert_array_equal(beta2[..., keep], beta[..., keep])
    np.testing.assert_array_equal(alpha2[..., keep], alpha[..., keep])
    assert np.abs(beta2[..., 1] - beta[..., 1]).max() > 1e-3
    assert np.abs(alpha2[..., 1] - alpha[..., 1]).max() > 1e-3


def _mean_of_sigmoids(x, w, b, beta_scale=1.0):
    x, w, b = (np.asarray(a, dtype=np.float64) for a in (x, w, b))
    H = w.shape[0] // 2
    z = x @ w.T
    return beta_scale / (1 + np.exp(-(z[..., :H] + b[:H]))), (1 / (1 + np.exp(-(z[..., H:] + b[H:])))).mean(axis=1)


def _rows_swapped(x, w, b, beta_scale=1.0):
    H = w.shape[0] // 2
    return _ORIG(x, np.concatenate([w[H:], w[:H]]), b, beta_scale)


def _scale_on_alpha(x, w, b, beta_scale=1.0):
    beta, alpha = _ORIG(x, w, b, 1.0)
    return beta, alpha * beta_scale


_ORIG = ora.gate_projections
MUTANTS = {"alpha as the mean of per-token sigmoids": _mean_of_sigmoids,
           "beta and alpha rows swapped": _rows_swapped,
           "beta_scale applied to alpha": _scale_on_alpha}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    monkeypatch.setattr(ora, "gate_projections", MUTANTS[name])
    failed = 0
    for pin in (test_brute_force_scalar_loops, test_zero_weights_give_the_biases,
                test_alpha_is_the_sigmoid_of_the_mean_logit, test_token_permutation):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, name
