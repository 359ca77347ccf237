"""ARL2 hybrid attention layer, forward hot path: the plain CPU oracle.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this module.  The product library never imports, links or
calls it, and it shares no code, table or constant with the HIP kernels.

Everything runs in numpy float64 (an fp32 mode exists for drift studies).  The inputs are
the values the GPU receives: bf16-representable Q, K, V and phi promoted to fp64, fp32 alpha
and beta promoted to fp64.

Sources.  [TS] is the technical summary "Attend Locally, Remember Linearly: Linear Attention
as Cross-Frame Memory for Autoregressive Video Diffusion" on gist.science (the German page;
the Italian, Japanese and Korean pages repeat it section by section).  [ABS] is the authors'
abstract of the same title as shown on fugumt.com.

What the layer computes, per stream b, head h and latent frame N, on the frame's T tokens
(rows of Q, K, V in R^{T x d}):

  O_intra = softmax(Q K^T / sqrt(d)) V             bidirectional within the frame [TS 2.1, intra branch]
  Q' = Q phi_q,  K' = unit_rows(K phi_k),  V' = V phi_v      per-head 1x1 maps [TS 2.1, adaptation]
  O = O_intra + Q' S_{N-1}                          same S_{N-1} for every token [TS 2.1 output; 2.2]
  S_N = alpha_N S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1})   once per frame [TS 2.1 state update; 2.2]

Readings taken where the pages leave a step open (each is also listed in the design notes):
  * the printed update has no transpose on the first K'; with token rows it must be K'^T for
    the shapes to conform and for O_inter = Q' S to read what the write stored;
  * alpha multiplies S_{N-1} only; the residual V' - K' S_{N-1} uses the undecayed state;
  * alpha is one scalar per (stream, frame, head); beta is one scalar per (stream, token, head);
  * the two branches are summed, with no gate, norm or output projection inside the layer;
  * softmax scale is 1/sqrt(d) (the pretrained layer's own attention);
  * the 1x1 maps use the row-vector convention x' = x phi, no bias, no activation;
  * K' rows are L2-normalised as k / max(||k||, eps), eps = 1e-6; Q' and V' are not;
  * S_0 = 0; denoising passes read S and never write it; the clean pass returns its output
    (computed with S_{N-1}) and then writes S_N [TS 2.2 clean-pass updates; ABS].
"""
from __future__ import annotations

import numpy as np

DEFAULT_KNORM_EPS = 1e-6


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Bidirectional softmax attention of one head over one frame's tokens.

    q, k, v: [T, d].  Row t of the result is sum_s p_ts v_s with p_t = softmax(scale * q_t . k_s)
    over all s of the same frame ([TS] 2.1, intra-frame branch).  Subtracting the row maximum
    before exp leaves the softmax unchanged and only avoids overflow."""
    a = (q @ k.T) * scale
    a = a - a.max(axis=1, keepdims=True)
    p = np.exp(a)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def feature_map(x: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """Per-head grouped 1x1 map applied to every token: x'[t, j] = sum_i x[t, i] phi[i, j]
    ([TS] 2.1, adaptation to the linear recurrence)."""
    return x @ phi


def unit_rows(x: np.ndarray, eps: float = DEFAULT_KNORM_EPS) -> np.ndarray:
    """Each row divided by max(its Euclidean norm, eps)."""
    n = np.sqrt(np.sum(x * x, axis=1, keepdims=True))
    return x / np.maximum(n, eps)


def inter_read(q_prime: np.ndarray, s: np.ndarray) -> np.ndarray:
    """O_inter = Q' S_{N-1}: every token reads the same state ([TS] 2.1 output; 2.2 frame-level
    access)."""
    return q_prime @ s


def gate_projections(x: np.ndarray, w_gates: np.ndarray, b_gates: np.ndarray, beta_scale: float = 1.0):
    """alpha and beta from the layer's hidden states ([TS] 2.1: the forget gate alpha and the
    learning rate beta are learned projections of the tokens; [TS] 4, ablations: head-wise gates).

    x [B, T, H d]; w_gates [2H, H d] (row h: beta of head h, row H + h: alpha of head h);
    b_gates [2H].  beta[b, t, h] = beta_scale * sigmoid(x[b, t] . w_gates[h] + b_gates[h]).
    The frame-level write applies one decay per (stream, head) and frame, so the per-token alpha
    logits are averaged over the frame's tokens before the sigmoid:
    alpha[b, h] = sigmoid(mean_t x[b, t] . w_gates[H + h] + b_gates[H + h]).
    Returns beta [B, T, H] and alpha [B, H]."""
    x = np.asarray(x, dtype=np.float64)
    w_gates = np.asarray(w_gates, dtype=np.float64)
    b_gates = np.asarray(b_gates, dtype=np.float64)
    H = w_gates.shape[0] // 2
    z = x @ w_gates.T  # [B, T, 2H] per-token logits
    beta = beta_scale / (1.0 + np.exp(-(z[..., :H] + b_gates[:H])))
    alpha = 1.0 / (1.0 + np.exp(-(z[..., H:].mean(axis=1) + b_gates[H:])))
    return beta, alpha


def delta_write(s: np.ndarray, k_prime: np.ndarray, v_prime: np.ndarray, beta: np.ndarray,
                alpha: float) -> np.ndarray:
    """Gated delta-rule frame write S_N = alpha S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1})
    ([TS] 2.1 state update), one write for the whole frame: every token's residual uses
    S_{N-1} ([TS] 2.2 frame-level access; [ABS])."""
    residual = v_prime - k_prime @ s
    return alpha * s + k_prime.T @ (beta[:, None] * residual)


class Arl2Oracle:
    """One ARL2 layer: fixed maps phi_q, phi_k, phi_v and a per-(stream, head) d x d state.

    Shapes follow the library's boundary: q, k, v [B, T, H, d]; beta [B, T, H]; alpha [B, H];
    phi_* [H, d, d]; state [B, H, d, d] (row index = key feature, column = value feature)."""

    def __init__(self, phi_q, phi_k, phi_v, batch: int, softmax_scale: float | None = None,
                 knorm_eps: float = DEFAULT_KNORM_EPS, dtype=np.float64):
        self.dtype = dtype
        self.phi_q = np.asarray(phi_q, dtype=dtype)
        self.phi_k = np.asarray(phi_k, dtype=dtype)
        self.phi_v = np.asarray(phi_v, dtype=dtype)
        heads, d, d2 = self.phi_q.shape
        if d != d2 or self.phi_k.shape != (heads, d, d) or self.phi_v.shape != (heads, d, d):
            raise ValueError("phi maps must be [H, d, d]")
        self.batch, self.heads, self.head_dim = batch, heads, d
        self.scale = (1.0 / np.sqrt(d)) if not softmax_scale else float(softmax_scale)
        self.eps = knorm_eps
        self.state = np.zeros((batch, heads, d, d), dtype=dtype)  # S_0 = 0
        self.frame = 0

    def _check(self, x: np.ndarray, name: str) -> np.ndarray:
        x = np.asarray(x, dtype=self.dtype)
        if x.ndim != 4 or x.shape[0] != self.batch or x.shape[2] != self.heads or x.shape[3] != self.head_dim:
            raise ValueError(f"{name} must be [B, T, H, d], got {x.shape}")
        return x

    def query(self, q, k, v) -> np.ndarray:
        """Output of one pass of the current frame with S_{N-1}; the state is not touched."""
        q, k, v = self._check(q, "q"), self._check(k, "k"), self._check(v, "v")
        out = np.empty(q.shape, dtype=self.dtype)
        for b in range(self.batch):
            for h in range(self.heads):
                o_intra = softmax_attention(q[b, :, h], k[b, :, h], v[b, :, h], self.scale)
                q_prime = feature_map(q[b, :, h], self.phi_q[h])
                out[b, :, h] = o_intra + inter_read(q_prime, self.state[b, h])
        return out

    def query_rows(self, q, k, v, rows) -> np.ndarray:
        """Outputs of the given token rows only ([B, len(rows), H, d]): query() restricted to a
        subset of query tokens, built from the same functions (softmax attention treats every
        query row on its own; keys and values stay complete)."""
        q, k, v = self._check(q, "q"), self._check(k, "k"), self._check(v, "v")
        rows = np.asarray(rows)
        out = np.empty((self.batch, len(rows), self.heads, self.head_dim), dtype=self.dtype)
        for b in range(self.batch):
            for h in range(self.heads):
                qr = q[b, rows, h]
                o_intra = softmax_attention(qr, k[b, :, h], v[b, :, h], self.scale)
                out[b, :, h] = o_intra + inter_read(feature_map(qr, self.phi_q[h]), self.state[b, h])
        return out

    denoise_step = query

    def next_state(self, k, v, beta, alpha) -> np.ndarray:
        """S_N from the clean pass's K, V and the frame's gates (does not commit it)."""
        k, v = self._check(k, "k"), self._check(v, "v")
        beta = np.asarray(beta, dtype=self.dtype)
        alpha = np.asarray(alpha, dtype=self.dtype)
        if beta.shape != k.shape[:3] or alpha.shape != (self.batch, self.heads):
            raise ValueError("beta must be [B, T, H] and alpha [B, H]")
        new = np.empty_like(self.state)
        for b in range(self.batch):
            for h in range(self.heads):
                k_prime = unit_rows(feature_map(k[b, :, h], self.phi_k[h]), self.eps)
                v_prime = feature_map(v[b, :, h], self.phi_v[h])
                new[b, h] = delta_write(self.state[b, h], k_prime, v_prime, beta[b, :, h], alpha[b, h])
        return new

    def commit(self, q, k, v, beta, alpha, want_output: bool = True):
        """Clean pass: output with S_{N-1} (optional), then write S_N once and advance."""
        out = self.query(q, k, v) if want_output else None
        self.state = self.next_state(k, v, beta, alpha)
        self.frame += 1
        return out
