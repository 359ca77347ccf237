"""Plant plausible mistakes in the oracle (CPU only) and check that the pins catch each one.

A pin set that still passes with a transposed map, a flipped sign or alpha in the wrong
place would not be pinning anything; this runs every golden and invariant pin against each
mutant and requires at least one failure.
"""
import inspect

import numpy as np
import pytest

import oracle.arl2_oracle as ora
from tests import test_oracle_golden as golden
from tests import test_oracle_invariants as inv


def _pins():
    fns = []
    for mod in (golden, inv):
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if name.startswith("test_") and fn.__module__ == mod.__name__:
                params = inspect.signature(fn).parameters
                if "alpha" in params:
                    fns += [(f"{name}[{a}]", (lambda f=fn, a=a: f(alpha=a))) for a in (0.0, 0.37, 1.0)]
                elif not params:
                    fns.append((name, fn))
    return fns


def _softmax_wrong_axis(q, k, v, scale):
    a = (q @ k.T) * scale
    p = np.exp(a - a.max(axis=0, keepdims=True))
    return (p / p.sum(axis=0, keepdims=True)) @ v


def _scale_one_over_d(q, k, v, scale):
    return ora.__dict__["_orig_softmax"](q, k, v, scale * scale)


MUTANTS = {
    "map transposed": ("feature_map", lambda x, phi: x @ phi.T),
    "softmax over keys axis swapped": ("softmax_attention", _softmax_wrong_axis),
    "scale 1/d": ("softmax_attention", _scale_one_over_d),
    "no key normalisation": ("unit_rows", lambda x, eps=1e-6: x),
    "no inter-frame read": ("inter_read", lambda qp, s: np.zeros((qp.shape[0], s.shape[1]))),
    "inter read with S^T": ("inter_read", lambda qp, s: qp @ s.T),
    "alpha inside residual": ("delta_write", lambda s, kp, vp, beta, alpha:
                              alpha * s + kp.T @ (beta[:, None] * (vp - alpha * (kp @ s)))),
    "residual sign flipped": ("delta_write", lambda s, kp, vp, beta, alpha:
                              alpha * s + kp.T @ (beta[:, None] * (vp + kp @ s))),
    "beta averaged over tokens": ("delta_write", lambda s, kp, vp, beta, alpha:
                                  alpha * s + kp.T @ (beta.mean() * (vp - kp @ s))),
    "alpha dropped": ("delta_write", lambda s, kp, vp, beta, alpha: s + kp.T @ (beta[:, None] * (vp - kp @ s))),
    "write transposed": ("delta_write", lambda s, kp, vp, beta, alpha:
                         (alpha * s + kp.T @ (beta[:, None] * (vp - kp @ s))).T),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, monkeypatch):
    name, fn = MUTANTS[mutant]
    monkeypatch.setitem(ora.__dict__, "_orig_softmax", ora.softmax_attention)
    monkeypatch.setattr(ora, name, fn)
    failed = []
    for pin_name, pin in _pins():
        try:
            pin()
        except (AssertionError, ValueError):
            failed.append(pin_name)
    assert failed, f"no pin caught the mutant '{mutant}'"


def test_output_after_write_is_caught(monkeypatch):
    """The clean pass computing its output with S_N instead of S_{N-1}."""
    def commit(self, q, k, v, beta, alpha, want_output=True):
        self.state = self.next_state(k, v, beta, alpha)
        self.frame += 1
        return self.query(q, k, v) if want_output else None

    monkeypatch.setattr(ora.Arl2Oracle, "commit", commit)
    with pytest.raises(AssertionError):
        inv.test_every_token_reads_the_same_pre_update_state()
