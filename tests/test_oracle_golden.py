"""The oracle against a two-frame example worked by hand (tests/golden/hand_example_d2.json)."""
import json
import math
import os

import numpy as np

from oracle import Arl2Oracle
from oracle.bruteforce import run_stream

HERE = os.path.dirname(os.path.abspath(__file__))
_NAMES = {"exp": math.exp, "sqrt": math.sqrt}


def _ev(expr):
    return eval(expr, {"__builtins__": {}}, _NAMES)  # closed-form expressions of the fixture only


def _load():
    with open(os.path.join(HERE, "golden", "hand_example_d2.json")) as f:
        return json.load(f)


def test_hand_example_vectorised_oracle():
    fx = _load()
    eye = np.eye(2)[None]
    orc = Arl2Oracle(eye, eye, eye, batch=1)
    for fr in fx["frames"]:
        q, k, v = (np.array(fr[n], dtype=np.float64)[None, :, None, :] for n in ("q", "k", "v"))
        beta = np.array(fr["beta"], dtype=np.float64)[None, :, None]
        alpha = np.array([[fr["alpha"]]])
        out = orc.commit(q, k, v, beta, alpha)
        want_o = np.array([[_ev(e) for e in row] for row in fr["expected_output"]])
        want_s = np.array([[_ev(e) for e in row] for row in fr["expected_state"]])
        np.testing.assert_allclose(out[0, :, 0, :], want_o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(orc.state[0, 0], want_s, rtol=0, atol=1e-13)


def test_hand_example_bruteforce():
    fx = _load()
    eye = np.eye(2)
    frames = [{"passes": [(fr["q"], fr["k"], fr["v"])], "beta": fr["beta"], "alpha": fr["alpha"]}
              for fr in fx["frames"]]
    outs, states = run_stream(eye, eye, eye, frames)
    for f, fr in enumerate(fx["frames"]):
        want_o = np.array([[_ev(e) for e in row] for row in fr["expected_output"]])
        want_s = np.array([[_ev(e) for e in row] for row in fr["expected_state"]])
        np.testing.assert_allclose(np.array(outs[f][0]), want_o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(np.array(states[f]), want_s, rtol=0, atol=1e-13)
