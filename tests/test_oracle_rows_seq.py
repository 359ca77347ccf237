"""Pins of the two oracle entry points that the sampled-row and token-level GPU parity tests rest
on (CPU only):

* ``Arl2Oracle.query_rows`` (outputs of selected token rows, used wherever a full frame is too
  large to recompute) must equal ``query()`` restricted to those rows: random, ragged, repeated
  and permuted row sets, several streams and heads, a non-zero state.
* ``Arl2SeqOracle.run`` / ``commit`` (the token-level access variant) must equal a scalar
  brute force of a two-frame stream with denoising and clean passes and alpha != 1, written in
  the other form of the clean write (decayed S_{N-1} plus the sum of the tokens' increments),
  and with one token per frame it must reduce to the frame-level layer.

Sources: "Attend Locally, Remember Linearly" technical summary (gist.science), section 2.1 (the
output Q'S_{N-1} added to the intra-frame softmax branch; the gated update) and section 2.2
(frame-level access, the alternative it rejects, one write per frame after the clean pass).
Each pin is also run against planted mistakes, every one of which must fail at least one pin.
"""
import numpy as np
import pytest

import oracle.arl2_oracle as ora
import oracle.seq_oracle as so
from oracle import Arl2Oracle, Arl2SeqOracle, feature_map, inter_read, softmax_attention, unit_rows
from oracle.bruteforce import seq_run_stream

RNG = np.random.default_rng(77)


def _maps(heads, d, scale=0.3):
    return [np.eye(d)[None] + scale * RNG.standard_normal((heads, d, d)) for _ in range(3)]


def _warm_layer(B=2, H=3, d=8, T=13):
    phis = _maps(H, d)
    orc = Arl2Oracle(*phis, batch=B)
    for _ in range(2):
        q, k, v = (RNG.standard_normal((B, T, H, d)) for _ in range(3))
        orc.commit(q, k, v, RNG.uniform(0.1, 0.9, (B, T, H)), RNG.uniform(0.4, 0.95, (B, H)))
    assert np.abs(orc.state).max() > 1e-2
    return orc


# --- query_rows ------------------------------------------------------------------------------

ROW_SETS = {
    "random subset": lambda T: np.sort(RNG.choice(T, size=min(5, T), replace=False)),
    "ragged ends": lambda T: np.array([0, T - 1]),
    "repeated rows": lambda T: np.array([3, 3, 7, 3, T - 1, T - 1]) % T,
    "all rows permuted": lambda T: RNG.permutation(T),
    "one row": lambda T: np.array([T // 2]),
}


def check_query_rows(orc=None, T=13):
    orc = orc or _warm_layer(T=T)
    B, H, d = orc.batch, orc.heads, orc.head_dim
    q, k, v = (RNG.standard_normal((B, T, H, d)) for _ in range(3))
    full = orc.query(q, k, v)
    for name, make in ROW_SETS.items():
        rows = make(T)
        got = orc.query_rows(q, k, v, rows)
        assert got.shape == (B, len(rows), H, d), name
        np.testing.assert_allclose(got, full[:, rows], rtol=0, atol=1e-13, err_msg=name)


@pytest.mark.parametrize("T", [1, 13, 40])
def test_query_rows_is_query_restricted_to_the_rows(T):
    check_query_rows(T=T)


def test_query_rows_with_zero_state_is_softmax_attention():
    """S_0 = 0: the rows' outputs are softmax attention of those queries over all keys."""
    B, H, d, T = 2, 2, 8, 11
    orc = Arl2Oracle(*_maps(H, d), batch=B)
    q, k, v = (RNG.standard_normal((B, T, H, d)) for _ in range(3))
    rows = np.array([1, 4, 10])
    got = orc.query_rows(q, k, v, rows)
    for b in range(B):
        for h in range(H):
            a = q[b, rows, h] @ k[b, :, h].T / np.sqrt(d)
            p = np.exp(a - a.max(axis=1, keepdims=True))
            want = (p / p.sum(axis=1, keepdims=True)) @ v[b, :, h]
            np.testing.assert_allclose(got[b, :, h], want, rtol=0, atol=1e-13)


def _rows_keys_restricted(self, q, k, v, rows):
    out = np.empty((self.batch, len(rows), self.heads, self.head_dim))
    for b in range(self.batch):
        for h in range(self.heads):
            qr = q[b, rows, h]
            out[b, :, h] = (softmax_attention(qr, k[b, rows, h], v[b, rows, h], self.scale)
                            + inter_read(feature_map(qr, self.phi_q[h]), self.state[b, h]))
    return out


def _rows_no_inter(self, q, k, v, rows):
    out = np.empty((self.batch, len(rows), self.heads, self.head_dim))
    for b in range(self.batch):
        for h in range(self.heads):
            out[b, :, h] = softmax_attention(q[b, rows, h], k[b, :, h], v[b, :, h], self.scale)
    return out


def _rows_state_transposed(self, q, k, v, rows):
    out = np.empty((self.batch, len(rows), self.heads, self.head_dim))
    for b in range(self.batch):
        for h in range(self.heads):
            qr = q[b, rows, h]
            out[b, :, h] = (softmax_attention(qr, k[b, :, h], v[b, :, h], self.scale)
                            + feature_map(qr, self.phi_q[h]) @ self.state[b, h].T)
    return out


def _rows_head_mixed(self, q, k, v, rows):
    out = np.empty((self.batch, len(rows), self.heads, self.head_dim))
    for b in range(self.batch):
        for h in range(self.heads):
            qr = q[b, rows, h]
            o = softmax_attention(qr, k[b, :, h], v[b, :, h], self.scale)
            out[b, :, h] = o + inter_read(feature_map(qr, self.phi_q[0]), self.state[b, h])
    return out


ROWS_MUTANTS = {"keys restricted to the rows": _rows_keys_restricted, "inter read dropped": _rows_no_inter,
                "state transposed": _rows_state_transposed, "head 0's map for every head": _rows_head_mixed}


@pytest.mark.parametrize("name", sorted(ROWS_MUTANTS))
def test_query_rows_pin_catches_mutant(name, monkeypatch):
    monkeypatch.setattr(ora.Arl2Oracle, "query_rows", ROWS_MUTANTS[name])
    with pytest.raises(AssertionError):
        check_query_rows()


# --- token-level access: run / commit ----------------------------------------------------------

def _seq_stream(B=2, H=2, d=4, T=5, frames=2, denoise=2):
    phis = _maps(H, d)
    data = []
    for _ in range(frames):
        passes = [tuple(RNG.standard_normal((B, T, H, d)) for _ in range(3)) for _ in range(denoise + 1)]
        data.append({"passes": passes, "beta": RNG.uniform(0.1, 0.9, (B, T, H)),
                     "alpha": RNG.uniform(0.3, 0.8, (B, H))})
    return phis, data


def check_seq_against_brute_force(B=2, H=2, d=4, T=5):
    phis, data = _seq_stream(B, H, d, T)
    orc = Arl2SeqOracle(*phis, batch=B)
    outs, states = [], []
    for fr in data:
        o = [orc.denoise_step(q, k, v, fr["beta"]) for (q, k, v) in fr["passes"][:-1]]
        o.append(orc.commit(*fr["passes"][-1], fr["beta"], fr["alpha"]))
        outs.append(o)
        states.append(orc.state.copy())
    for b in range(B):
        for h in range(H):
            frames = [{"passes": [(q[b, :, h], k[b, :, h], v[b, :, h]) for (q, k, v) in fr["passes"]],
                       "beta": fr["beta"][b, :, h], "alpha": fr["alpha"][b, h]} for fr in data]
            bf_out, bf_state = seq_run_stream(phis[0][h], phis[1][h], phis[2][h], frames)
            for f in range(len(data)):
                for p in range(len(data[f]["passes"])):
                    np.testing.assert_allclose(outs[f][p][b, :, h], np.array(bf_out[f][p]), rtol=0, atol=1e-12)
                np.testing.assert_allclose(states[f][b, h], np.array(bf_state[f]), rtol=0, atol=1e-12)


def test_seq_oracle_equals_brute_force():
    check_seq_against_brute_force()


def check_seq_one_token_is_frame_level(B=2, H=2, d=6):
    """With one token per frame there is nothing to order: the token-level layer's outputs and
    state equal the frame-level layer's, frame after frame."""
    phis = _maps(H, d)
    seq, frame = Arl2SeqOracle(*phis, batch=B), Arl2Oracle(*phis, batch=B)
    for _ in range(3):
        q, k, v = (RNG.standard_normal((B, 1, H, d)) for _ in range(3))
        beta, alpha = RNG.uniform(0.1, 0.9, (B, 1, H)), RNG.uniform(0.3, 0.8, (B, H))
        np.testing.assert_allclose(seq.denoise_step(q, k, v, beta), frame.denoise_step(q, k, v), rtol=0, atol=1e-13)
        np.testing.assert_allclose(seq.commit(q, k, v, beta, alpha), frame.commit(q, k, v, beta, alpha),
                                   rtol=0, atol=1e-13)
        np.testing.assert_allclose(seq.state, frame.state, rtol=0, atol=1e-13)


def test_seq_one_token_is_frame_level():
    check_seq_one_token_is_frame_level()


def test_seq_denoise_passes_never_write():
    phis, data = _seq_stream()
    orc = Arl2SeqOracle(*phis, batch=2)
    orc.commit(*data[0]["passes"][-1], data[0]["beta"], data[0]["alpha"])
    before = orc.state.copy()
    for (q, k, v) in data[1]["passes"]:
        orc.denoise_step(q, k, v, data[1]["beta"])
    assert np.array_equal(orc.state, before) and orc.frame == 1


def _run_template(alpha_on_final=False, drop_softmax=False, decay_inside=False, denoise_writes=False):
    def run(self, q, k, v, beta, alpha=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        beta = np.asarray(beta, dtype=np.float64)
        out = np.empty_like(q)
        new = np.empty_like(self.state)
        for b in range(self.batch):
            for h in range(self.heads):
                qp = feature_map(q[b, :, h], self.phi_q[h])
                kp = unit_rows(feature_map(k[b, :, h], self.phi_k[h]), self.eps)
                vp = feature_map(v[b, :, h], self.phi_v[h])
                a = 1.0 if alpha is None else float(np.asarray(alpha)[b, h])
                start = a * self.state[b, h] if decay_inside else self.state[b, h]
                o_inter, s_t = so.sequential_frame(qp, kp, vp, beta[b, :, h], start)
                o_sm = softmax_attention(q[b, :, h], k[b, :, h], v[b, :, h], self.scale)
                out[b, :, h] = o_inter if drop_softmax else o_sm + o_inter
                if alpha_on_final:
                    new[b, h] = a * s_t
                elif decay_inside:
                    new[b, h] = s_t
                else:
                    new[b, h] = s_t - (1.0 - a) * self.state[b, h]
        if alpha is None and not denoise_writes:
            return out, None
        return out, new

    if denoise_writes:
        def denoise_step(self, q, k, v, beta):
            out, new = run(self, q, k, v, beta)
            self.state = new
            return out
        return run, denoise_step
    return run, None


SEQ_MUTANTS = {
    "alpha applied to S^(T)": dict(alpha_on_final=True),
    "softmax branch dropped": dict(drop_softmax=True),
    "decay applied before the recurrence": dict(decay_inside=True),
    "denoising pass writes the state": dict(denoise_writes=True),
}


@pytest.mark.parametrize("name", sorted(SEQ_MUTANTS))
def test_seq_pins_catch_mutant(name, monkeypatch):
    run, denoise = _run_template(**SEQ_MUTANTS[name])
    monkeypatch.setattr(so.Arl2SeqOracle, "run", run)
    if denoise is not None:
        monkeypatch.setattr(so.Arl2SeqOracle, "denoise_step", denoise)
    failed = 0
    for pin in (check_seq_against_brute_force, check_seq_one_token_is_frame_level):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, name
