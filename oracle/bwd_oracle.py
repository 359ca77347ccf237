"""Backward of the ARL2 layer: gradients through its passes, its state write and across frames.
The plain CPU oracle.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this module.  The product library never imports, links or
calls it, and it shares no code, table or constant with the HIP kernels.

numpy float64; inputs are the values the GPU receives.

Source.  [TS] technical summary "Attend Locally, Remember Linearly" (gist.science): section 2.1
and 2.2 define the forward whose gradients are taken here; section 2.3 trains the converted
model by distillation, the second stage end to end through every replaced layer, with the
per-head maps (and gates) as the trainable parameters.  The pages print no backward: every
formula below is the chain rule applied to the forward of the frame-level oracle
(``oracle.arl2_oracle``), written out per term.

Forward of frame N for one (stream, head), passes p = 0..P (the last is the clean pass, whose
K, V and gates write the state):
  out_p = softmax(scale Q_p K_p^T) V_p + (Q_p phi_q) S_{N-1}
  S_N   = alpha S_{N-1} + K'^T diag(beta) R,   R = V' - K' S_{N-1},
          K' = unit_rows(K phi_k), V' = V phi_v          (K, V of the clean pass)
Given dO_p = dL/d out_p for each pass and G = dL/dS_N, the reverse sweep over frames returns
dL/dQ_p, dL/dK_p, dL/dV_p, dL/dbeta, dL/dalpha, dL/dS_{N-1} and adds to dL/dphi_q, dL/dphi_k,
dL/dphi_v:
  softmax branch:  P = softmax rows of scale Q K^T;  dV = P^T dO;  dP = dO V^T;
                   dA = P o (dP - rowsum(P o dP));  dQ = scale dA K;  dK = scale dA^T Q
  inter-frame read (out += Q phi_q S):  dQ' = dO S^T;  dQ += dQ' phi_q^T;
                   dphi_q += Q^T dQ';  dS_{N-1} += (Q phi_q)^T dO
  state write:     X = K' G;  dR = diag(beta) X;  dbeta_t = x_t . r_t;  dalpha = <G, S_{N-1}>;
                   dK' = diag(beta) R G^T - dR S_{N-1}^T;  dV' = dR;
                   dS_{N-1} += alpha G - K'^T dR
  maps:            dV += dV' phi_v^T, dphi_v += V^T dV';  for K' = U / max(|U|, eps), U = K phi_k:
                   dU_t = (dK'_t - k'_t (k'_t . dK'_t)) / |u_t| where |u_t| > eps, else dK'_t / eps;
                   dK += dU phi_k^T, dphi_k += K^T dU
Readings: which passes enter the loss is the trainer's choice (a pass without an output
gradient contributes nothing); alpha and beta are taken as inputs, so their gradients are
returned as such (the gate projections that produce them are ordinary linear layers of the
caller); at |u_t| = eps exactly the constant branch of the max is taken.
"""
from __future__ import annotations

import numpy as np

from .arl2_oracle import DEFAULT_KNORM_EPS, delta_write, feature_map, unit_rows


def softmax_attention_bwd(q, k, v, d_o, scale):
    """Gradients of sum <d_o, softmax(scale q k^T) v> with respect to q, k, v ([T, d] each)."""
    a = (q @ k.T) * scale
    a = a - a.max(axis=1, keepdims=True)
    p = np.exp(a)
    p = p / p.sum(axis=1, keepdims=True)
    dv = p.T @ d_o
    dp = d_o @ v.T
    da = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    return scale * (da @ k), scale * (da.T @ q), dv


def inter_read_bwd(q, d_o, s_prev, phi_q):
    """out = (q phi_q) s_prev: gradients with respect to q, phi_q and s_prev."""
    dqp = d_o @ s_prev.T
    return dqp @ phi_q.T, q.T @ dqp, feature_map(q, phi_q).T @ d_o


def unit_rows_bwd(x, dy, eps=DEFAULT_KNORM_EPS):
    """y = x / max(|x|, eps) row by row: the gradient with respect to x given dy."""
    n = np.sqrt(np.sum(x * x, axis=1, keepdims=True))
    y = x / np.maximum(n, eps)
    big = n > eps
    proj = (dy - y * np.sum(y * dy, axis=1, keepdims=True)) / np.where(big, n, 1.0)
    return np.where(big, proj, dy / eps)


def delta_write_bwd(s_prev, k_prime, v_prime, beta, alpha, g):
    """S_N = alpha s_prev + K'^T diag(beta) (V' - K' s_prev), given G = dL/dS_N: returns
    (dS_{N-1} from the write, dK', dV', dbeta [T], dalpha)."""
    r = v_prime - k_prime @ s_prev
    x = k_prime @ g
    dr = beta[:, None] * x
    dk_prime = beta[:, None] * (r @ g.T) - dr @ s_prev.T
    ds = alpha * g - k_prime.T @ dr
    return ds, dk_prime, dr, np.sum(x * r, axis=1), float(np.sum(g * s_prev))


def pass_backward(q, k, v, d_o, s_prev, phi_q, scale):
    """One pass of one frame, all streams and heads.  q, k, v, d_o [B, T, H, d]; s_prev
    [B, H, d, d]; phi_q [H, d, d].  Returns dq, dk, dv [B, T, H, d], dS_{N-1} contribution
    [B, H, d, d] and dphi_q contribution [H, d, d]."""
    q, k, v, d_o = (np.asarray(x, dtype=np.float64) for x in (q, k, v, d_o))
    B, T, H, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    ds = np.zeros((B, H, d, d))
    dphi = np.zeros((H, d, d))
    for b in range(B):
        for h in range(H):
            a, bk, c = softmax_attention_bwd(q[b, :, h], k[b, :, h], v[b, :, h], d_o[b, :, h], scale)
            ri, rphi, rs = inter_read_bwd(q[b, :, h], d_o[b, :, h], s_prev[b, h], phi_q[h])
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = a + ri, bk, c
            ds[b, h] = rs
            dphi[h] += rphi
    return dq, dk, dv, ds, dphi


def write_backward(k, v, beta, alpha, s_prev, g, phi_k, phi_v, eps=DEFAULT_KNORM_EPS):
    """The state write of one frame, all streams and heads.  k, v [B, T, H, d] (clean pass);
    beta [B, T, H]; alpha [B, H]; s_prev, g [B, H, d, d].  Returns dk, dv, dbeta, dalpha,
    dS_{N-1} contribution, dphi_k and dphi_v contributions."""
    k, v = np.asarray(k, dtype=np.float64), np.asarray(v, dtype=np.float64)
    B, T, H, d = k.shape
    dk, dv = np.zeros_like(k), np.zeros_like(v)
    dbeta, dalpha = np.zeros((B, T, H)), np.zeros((B, H))
    ds = np.zeros((B, H, d, d))
    dphi_k, dphi_v = np.zeros((H, d, d)), np.zeros((H, d, d))
    for b in range(B):
        for h in range(H):
            u = feature_map(k[b, :, h], phi_k[h])
            kp = unit_rows(u, eps)
            vp = feature_map(v[b, :, h], phi_v[h])
            ds[b, h], dkp, dvp, dbeta[b, :, h], dalpha[b, h] = delta_write_bwd(
                s_prev[b, h], kp, vp, beta[b, :, h], float(alpha[b, h]), g[b, h])
            du = unit_rows_bwd(u, dkp, eps)
            dk[b, :, h], dv[b, :, h] = du @ phi_k[h].T, dvp @ phi_v[h].T
            dphi_k[h] += k[b, :, h].T @ du
            dphi_v[h] += v[b, :, h].T @ dvp
    return dk, dv, dbeta, dalpha, ds, dphi_k, dphi_v


def forward_states(phi_k, phi_v, frames, s0, eps=DEFAULT_KNORM_EPS):
    """S_0 .. S_F of a stream of frames (each a dict with 'passes' [(q, k, v), ...], clean last,
    'beta' [B, T, H], 'alpha' [B, H])."""
    states = [np.array(s0, dtype=np.float64)]
    for fr in frames:
        _, k, v = (np.asarray(x, dtype=np.float64) for x in fr["passes"][-1])
        s = states[-1]
        B, _, H, _ = k.shape
        new = np.empty_like(s)
        for b in range(B):
            for h in range(H):
                new[b, h] = delta_write(s[b, h], unit_rows(feature_map(k[b, :, h], phi_k[h]), eps),
                                        feature_map(v[b, :, h], phi_v[h]), np.asarray(fr["beta"])[b, :, h],
                                        float(np.asarray(fr["alpha"])[b, h]))
        states.append(new)
    return states


def layer_backward(phi_q, phi_k, phi_v, frames, d_outs, g_last=None, s0=None, scale=None,
                   eps=DEFAULT_KNORM_EPS):
    """Gradients of a stream of frames.  frames as in forward_states; d_outs[N][p]: dO of pass p
    of frame N ([B, T, H, d]) or None; g_last: dL/dS_F (zero if None); s0: S_0 (zero if None).
    Returns a dict: 'dq', 'dk', 'dv' (lists per frame of lists per pass), 'dbeta', 'dalpha'
    (lists per frame), 'dphi_q', 'dphi_k', 'dphi_v' [H, d, d], 'ds0' [B, H, d, d]."""
    phi_q, phi_k, phi_v = (np.asarray(p, dtype=np.float64) for p in (phi_q, phi_k, phi_v))
    H, d, _ = phi_q.shape
    B = np.asarray(frames[0]["passes"][0][0]).shape[0]
    scale = 1.0 / np.sqrt(d) if not scale else float(scale)
    s0 = np.zeros((B, H, d, d)) if s0 is None else np.asarray(s0, dtype=np.float64)
    states = forward_states(phi_k, phi_v, frames, s0, eps)
    g = np.zeros((B, H, d, d)) if g_last is None else np.array(g_last, dtype=np.float64)
    res = {"dq": [None] * len(frames), "dk": [None] * len(frames), "dv": [None] * len(frames),
           "dbeta": [None] * len(frames), "dalpha": [None] * len(frames),
           "dphi_q": np.zeros((H, d, d)), "dphi_k": np.zeros((H, d, d)), "dphi_v": np.zeros((H, d, d))}
    for n in range(len(frames) - 1, -1, -1):
        fr, s_prev = frames[n], states[n]
        dq_n, dk_n, dv_n = [], [], []
        g_prev = np.zeros_like(g)
        for p, (q, k, v) in enumerate(fr["passes"]):
            d_o = d_outs[n][p]
            if d_o is None:
                z = np.zeros(np.asarray(q).shape)
                dq_n.append(z), dk_n.append(z.copy()), dv_n.append(z.copy())
                continue
            a, bk, c, ds, dphi = pass_backward(q, k, v, d_o, s_prev, phi_q, scale)
            dq_n.append(a), dk_n.append(bk), dv_n.append(c)
            g_prev += ds
            res["dphi_q"] += dphi
        _, k, v = fr["passes"][-1]
        wk, wv, dbeta, dalpha, ds, dpk, dpv = write_backward(k, v, fr["beta"], fr["alpha"], s_prev, g,
                                                             phi_k, phi_v, eps)
        dk_n[-1] = dk_n[-1] + wk
        dv_n[-1] = dv_n[-1] + wv
        res["dq"][n], res["dk"][n], res["dv"][n] = dq_n, dk_n, dv_n
        res["dbeta"][n], res["dalpha"][n] = dbeta, dalpha
        res["dphi_k"] += dpk
        res["dphi_v"] += dpv
        g = g_prev + ds
    res["ds0"] = g
    return res
