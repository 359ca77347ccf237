"""ARL2 layer by scalar loops, one token and one state element at a time.

TEST INFRASTRUCTURE (same restrictions as ``arl2_oracle``).  This is the brute-force
recomputation the vectorised oracle is checked against on tiny inputs: pure Python floats
(IEEE double), no matrix routine, every sum written out.  It follows the same sources and
readings as ``arl2_oracle`` ([TS] 2.1 and 2.2 of "Attend Locally, Remember Linearly").
"""
from __future__ import annotations

import math


def _lists(x):
    return x.tolist() if hasattr(x, "tolist") else x


def token_output(q, k, v, phi_q, s, t, scale):
    """o_t for one head: softmax-weighted sum over the frame's keys plus (q_t phi_q) S."""
    T, d = len(k), len(q[0])
    scores = [scale * sum(q[t][i] * k[u][i] for i in range(d)) for u in range(T)]
    m = max(scores)
    w = [math.exp(x - m) for x in scores]
    z = sum(w)
    o = [sum(w[u] * v[u][j] for u in range(T)) / z for j in range(d)]
    qp = [sum(q[t][i] * phi_q[i][j] for i in range(d)) for j in range(d)]
    return [o[j] + sum(qp[i] * s[i][j] for i in range(d)) for j in range(d)]


def state_element(k, v, phi_k, phi_v, s, beta, alpha, i, j, eps):
    """S_N[i][j] = alpha S[i][j] + sum_t beta_t K'[t][i] (V'[t][j] - sum_l K'[t][l] S[l][j])."""
    T, d = len(k), len(k[0])
    acc = alpha * s[i][j]
    for t in range(T):
        kp = [sum(k[t][a] * phi_k[a][c] for a in range(d)) for c in range(d)]
        norm = math.sqrt(sum(x * x for x in kp))
        kp = [x / max(norm, eps) for x in kp]
        vp_j = sum(v[t][a] * phi_v[a][j] for a in range(d))
        pred_j = sum(kp[l] * s[l][j] for l in range(d))
        acc += beta[t] * kp[i] * (vp_j - pred_j)
    return acc


def run_stream(phi_q, phi_k, phi_v, frames, scale=None, eps=1e-6):
    """Run a whole stream for ONE stream and ONE head.

    phi_*: [d][d]; frames: list of dicts with 'passes' (list of (q, k, v), each [T][d]; the
    last pass is the clean pass), 'beta' [T] and 'alpha' (float).
    Returns (outputs, states): outputs[f][p] is [T][d]; states[f] is S after frame f."""
    phi_q, phi_k, phi_v = _lists(phi_q), _lists(phi_k), _lists(phi_v)
    d = len(phi_q)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = [[0.0] * d for _ in range(d)]
    outputs, states = [], []
    for fr in frames:
        outs = []
        for (q, k, v) in fr["passes"]:
            q, k, v = _lists(q), _lists(k), _lists(v)
            outs.append([token_output(q, k, v, phi_q, s, t, scale) for t in range(len(q))])
        _, kc, vc = (_lists(x) for x in fr["passes"][-1])
        beta = _lists(fr["beta"])
        s = [[state_element(kc, vc, phi_k, phi_v, s, beta, float(fr["alpha"]), i, j, eps)
              for j in range(d)] for i in range(d)]
        outputs.append(outs)
        states.append(s)
    return outputs, states


def seq_run_stream(phi_q, phi_k, phi_v, frames, scale=None, eps=1e-6):
    """The token-level (sequential) access variant for ONE stream and ONE head, by scalar loops
    (the alternative to frame-level access that [TS] 2.2 rejects: each token reads, and takes its
    residual against, the state the frame's earlier tokens have written).

    Same frame format as run_stream.  Every pass computes o_t = softmax branch_t + q'_t S^(t-1)
    with S^(0) = S_{N-1}; the clean pass then writes the frame's state as the decayed previous
    state plus the sum of the tokens' increments,
      S_N[i][j] = alpha S_{N-1}[i][j] + sum_t beta_t k'_t[i] (v'_t[j] - sum_l k'_t[l] S^(t-1)[l][j]),
    the increments being the ones the running state took.  Denoising passes write nothing.
    Returns (outputs, states) as run_stream."""
    phi_q, phi_k, phi_v = _lists(phi_q), _lists(phi_k), _lists(phi_v)
    d = len(phi_q)
    scale = 1.0 / math.sqrt(d) if scale is None else scale

    def mapped(x, phi):
        return [sum(x[a] * phi[a][c] for a in range(d)) for c in range(d)]

    s_prev = [[0.0] * d for _ in range(d)]
    outputs, states = [], []
    for fr in frames:
        beta = _lists(fr["beta"])
        outs, incr = [], None
        for p, (q, k, v) in enumerate(fr["passes"]):
            q, k, v = _lists(q), _lists(k), _lists(v)
            T = len(q)
            run = [row[:] for row in s_prev]  # S^(t-1), starting at S_{N-1}
            incr = [[0.0] * d for _ in range(d)]  # sum of the increments so far
            out = []
            for t in range(T):
                scores = [scale * sum(q[t][i] * k[u][i] for i in range(d)) for u in range(T)]
                m = max(scores)
                w = [math.exp(x - m) for x in scores]
                z = sum(w)
                qp = mapped(q[t], phi_q)
                out.append([sum(w[u] * v[u][j] for u in range(T)) / z + sum(qp[i] * run[i][j] for i in range(d))
                            for j in range(d)])
                kp = mapped(k[t], phi_k)
                norm = math.sqrt(sum(x * x for x in kp))
                kp = [x / max(norm, eps) for x in kp]
                vp = mapped(v[t], phi_v)
                resid = [vp[j] - sum(kp[l] * run[l][j] for l in range(d)) for j in range(d)]
                for i in range(d):
                    for j in range(d):
                        dlt = beta[t] * kp[i] * resid[j]
                        run[i][j] += dlt
                        incr[i][j] += dlt
            outs.append(out)
        alpha = float(fr["alpha"])
        s_prev = [[alpha * s_prev[i][j] + incr[i][j] for j in range(d)] for i in range(d)]
        outputs.append(outs)
        states.append(s_prev)
    return outputs, states
