"""Pins of the token-level (sequential) access oracle (CPU only): the chunked WY form of the
delta rule against the token loop, reductions to the frame-level write (one token; mutually
orthogonal keys), delta-rule retrieval, dependence on token order (the frame-level layer's
permutation equivariance fails here), and planted mistakes.

Sources: "Attend Locally, Remember Linearly" technical summary (gist.science), section 2.2
(frame-level access) and section 4 (experimental results, ablations); the authors' abstract.
"""
import numpy as np
import pytest

import oracle.seq_oracle as so
from oracle import delta_write, inter_read, unit_rows

RNG = np.random.default_rng(2024)


def _frame(T=7, d=6, beta_scale=0.5):
    qp = RNG.standard_normal((T, d))
    kp = unit_rows(RNG.standard_normal((T, d)))
    vp = RNG.standard_normal((T, d))
    beta = RNG.uniform(0.1, 1.0, T) * beta_scale
    s = RNG.standard_normal((d, d)) * 0.3
    return qp, kp, vp, beta, s


@pytest.mark.parametrize("chunk", [1, 3, 4, 7, 16])
def test_chunked_wy_form_equals_the_token_loop(chunk):
    qp, kp, vp, beta, s = _frame(T=11)
    o1, s1 = so.sequential_frame(qp, kp, vp, beta, s)
    o2, s2 = so.sequential_frame_chunked(qp, kp, vp, beta, s, chunk=chunk)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s2, s1, rtol=0, atol=1e-12)


def test_one_token_is_the_frame_level_write():
    qp, kp, vp, beta, s = _frame(T=1)
    o, s_t = so.sequential_frame(qp, kp, vp, beta, s)
    np.testing.assert_allclose(o, inter_read(qp, s), rtol=0, atol=1e-14)
    for alpha in (0.3, 1.0):
        np.testing.assert_allclose(s_t - (1 - alpha) * s, delta_write(s, kp, vp, beta, alpha), rtol=0, atol=1e-14)


def test_orthogonal_keys_give_the_frame_level_state():
    d = 8
    qp, _, vp, beta, s = _frame(T=5, d=d)
    kp = np.linalg.qr(RNG.standard_normal((d, d)))[0][:5]  # 5 orthonormal key rows
    _, s_t = so.sequential_frame(qp, kp, vp, beta, s)
    np.testing.assert_allclose(s_t - 0.4 * s, delta_write(s, kp, vp, beta, 0.6), rtol=0, atol=1e-13)


def test_delta_rule_retrieval():
    """With beta = 1 and unit keys, right after token t the running state returns v'_t at k'_t."""
    qp, kp, vp, _, s = _frame(T=6)
    beta = np.ones(6)
    for t in range(1, 7):
        _, s_t = so.sequential_frame(qp[:t], kp[:t], vp[:t], beta[:t], s)
        np.testing.assert_allclose(kp[t - 1] @ s_t, vp[t - 1], rtol=0, atol=1e-12)


def test_token_order_matters():
    """Permuting the tokens (with their queries, keys, values and betas) does not permute the
    outputs, nor leave the state, as the frame-level layer does: the asymmetry the pages avoid."""
    qp, kp, vp, beta, s = _frame(T=8)
    perm = RNG.permutation(8)
    o, s_t = so.sequential_frame(qp, kp, vp, beta, s)
    op, sp = so.sequential_frame(qp[perm], kp[perm], vp[perm], beta[perm], s)
    assert np.abs(op - o[perm]).max() > 1e-3
    assert np.abs(sp - s_t).max() > 1e-3


def test_first_token_reads_the_previous_state():
    qp, kp, vp, beta, s = _frame(T=5)
    o, _ = so.sequential_frame(qp, kp, vp, beta, s)
    np.testing.assert_allclose(o[0], qp[0] @ s, rtol=0, atol=1e-14)


# --- planted mistakes ----------------------------------------------------------------------

def _read_after_update(qp, kp, vp, beta, s_prev):
    s = np.array(s_prev, dtype=np.float64, copy=True)
    o = np.empty((qp.shape[0], s.shape[1]))
    for t in range(qp.shape[0]):
        s = s + beta[t] * np.outer(kp[t], vp[t] - kp[t] @ s)
        o[t] = qp[t] @ s
    return o, s


def _residual_against_frame_start(qp, kp, vp, beta, s_prev):
    s = np.array(s_prev, dtype=np.float64, copy=True)
    o = np.empty((qp.shape[0], s.shape[1]))
    for t in range(qp.shape[0]):
        o[t] = qp[t] @ s
        s = s + beta[t] * np.outer(kp[t], vp[t] - kp[t] @ s_prev)
    return o, s


def _key_transposed(qp, kp, vp, beta, s_prev):
    s = np.array(s_prev, dtype=np.float64, copy=True)
    o = np.empty((qp.shape[0], s.shape[1]))
    for t in range(qp.shape[0]):
        o[t] = qp[t] @ s
        s = s + beta[t] * np.outer(vp[t] - kp[t] @ s, kp[t])
    return o, s


MUTANTS = {"read after the update": _read_after_update,
           "residual against the frame's starting state": _residual_against_frame_start,
           "outer product transposed": _key_transposed}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    monkeypatch.setattr(so, "sequential_frame", MUTANTS[name])
    failed = 0
    pins = [lambda: test_chunked_wy_form_equals_the_token_loop(3), test_one_token_is_the_frame_level_write,
            test_delta_rule_retrieval, test_first_token_reads_the_previous_state]
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, name
