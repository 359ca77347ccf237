"""Token-level (sequential) access variant of the ARL2 layer: the plain CPU oracle.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this module.  The product library never imports, links or
calls it, and it shares no code, table or constant with the HIP kernels.

numpy float64; inputs are the values the GPU receives.

Source.  [TS] technical summary "Attend Locally, Remember Linearly" (gist.science), section 2.2
(frame-level access: every token of a frame reads the same pre-update state, to avoid an
information asymmetry inside the frame) and the ablations of section 4 (experimental results); [ABS] the authors'
abstract, which makes the same choice against updating the state token by token.  This module
is the alternative those passages reject, built as an A/B of the frame-level design.

Per stream b, head h and frame N, with Q' = Q phi_q, K' = unit_rows(K phi_k), V' = V phi_v
(the maps of the frame-level layer) and the frame's tokens t = 1..T in order:

  S^(0) = S_{N-1}
  o_t   = softmax branch_t + q'_t S^(t-1)                          (token t sees tokens < t)
  S^(t) = S^(t-1) + beta_t k'_t^T (v'_t - k'_t S^(t-1))            (residual against the running state)
  clean pass:  S_N = S^(T) - (1 - alpha) S_{N-1}
             = alpha S_{N-1} + sum_t beta_t k'_t^T (v'_t - k'_t S^(t-1))

Readings (the pages name the variant, not its formula): the frame-level write with each
token's residual and read taken against the running state instead of S_{N-1}; alpha decays
S_{N-1} once per frame exactly as in the frame-level write; denoising passes run the same
recurrence for their outputs and write nothing.  With T = 1, or with mutually orthogonal keys,
S_N equals the frame-level write; the outputs depend on token order (the frame-level layer's
permutation equivariance fails here).
"""
from __future__ import annotations

import numpy as np

from .arl2_oracle import DEFAULT_KNORM_EPS, feature_map, softmax_attention, unit_rows


def sequential_frame(q_prime, k_prime, v_prime, beta, s_prev):
    """The token-by-token recurrence of one (stream, head) frame: returns the inter-frame reads
    O_inter [T, d] (row t = q'_t S^(t-1)) and S^(T).  A plain loop over tokens."""
    s = np.array(s_prev, dtype=np.float64, copy=True)
    o = np.empty((q_prime.shape[0], s.shape[1]))
    for t in range(q_prime.shape[0]):
        o[t] = q_prime[t] @ s
        r = v_prime[t] - k_prime[t] @ s
        s = s + beta[t] * np.outer(k_prime[t], r)
    return o, s


def sequential_frame_chunked(q_prime, k_prime, v_prime, beta, s_prev, chunk: int = 4):
    """The same recurrence in chunks of `chunk` tokens (the WY form of the delta rule): per
    chunk, with A = I + strictly_lower(diag(beta) K K^T) and T = A^-1, the corrected values
    U_hat = T diag(beta) (V - K S) give O = Q S + strictly_lower(Q K^T) U_hat and
    S <- S + K^T U_hat.  Exact rewrite of the loop (a pin for it)."""
    s = np.array(s_prev, dtype=np.float64, copy=True)
    out = np.empty((q_prime.shape[0], s.shape[1]))
    for c0 in range(0, q_prime.shape[0], chunk):
        q, k, v, bt = (x[c0:c0 + chunk] for x in (q_prime, k_prime, v_prime, beta))
        a = np.eye(len(k)) + np.tril(bt[:, None] * (k @ k.T), -1)
        u_hat = np.linalg.solve(a, bt[:, None] * (v - k @ s))
        out[c0:c0 + chunk] = q @ s + np.tril(q @ k.T, -1) @ u_hat
        s = s + k.T @ u_hat
    return out, s


class Arl2SeqOracle:
    """The layer with token-level access.  Shapes as the frame-level oracle: q, k, v [B, T, H, d];
    beta [B, T, H]; alpha [B, H]; phi_* [H, d, d]; state [B, H, d, d]."""

    def __init__(self, phi_q, phi_k, phi_v, batch: int, softmax_scale: float | None = None,
                 knorm_eps: float = DEFAULT_KNORM_EPS):
        self.phi_q, self.phi_k, self.phi_v = (np.asarray(p, dtype=np.float64) for p in (phi_q, phi_k, phi_v))
        heads, d, _ = self.phi_q.shape
        self.batch, self.heads, self.head_dim = batch, heads, d
        self.scale = (1.0 / np.sqrt(d)) if not softmax_scale else float(softmax_scale)
        self.eps = knorm_eps
        self.state = np.zeros((batch, heads, d, d))
        self.frame = 0

    def run(self, q, k, v, beta, alpha=None):
        """One pass: (outputs [B, T, H, d], S_N or None).  S_N only when alpha is given."""
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        beta = np.asarray(beta, dtype=np.float64)
        out = np.empty_like(q)
        new = np.empty_like(self.state) if alpha is not None else None
        for b in range(self.batch):
            for h in range(self.heads):
                qp = feature_map(q[b, :, h], self.phi_q[h])
                kp = unit_rows(feature_map(k[b, :, h], self.phi_k[h]), self.eps)
                vp = feature_map(v[b, :, h], self.phi_v[h])
                o_inter, s_t = sequential_frame(qp, kp, vp, beta[b, :, h], self.state[b, h])
                out[b, :, h] = softmax_attention(q[b, :, h], k[b, :, h], v[b, :, h], self.scale) + o_inter
                if new is not None:
                    new[b, h] = s_t - (1.0 - float(np.asarray(alpha)[b, h])) * self.state[b, h]
        return out, new

    def denoise_step(self, q, k, v, beta):
        return self.run(q, k, v, beta)[0]

    def commit(self, q, k, v, beta, alpha):
        out, new = self.run(q, k, v, beta, alpha)
        self.state = new
        self.frame += 1
        return out
