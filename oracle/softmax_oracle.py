"""Retained softmax attention layer with a growing K/V cache: the plain CPU oracle.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this module.  The product library never imports, links or
calls it, and it shares no code, table or constant with the HIP kernels.

numpy float64 throughout; the inputs are the values the GPU receives (bf16-representable
Q, K, V promoted to fp64).

Sources.  [TS] is the technical summary "Attend Locally, Remember Linearly: Linear Attention
as Cross-Frame Memory for Autoregressive Video Diffusion" on gist.science: section 1 (the
problem) describes autoregressive video DiTs whose softmax self-attention keeps a key-value
cache that grows by one block per generated frame, and section 2 keeps softmax attention in
the layers the conversion does not replace; section 4 compares the hybrid model's memory and
speed with that baseline.  [ABS] is the authors' abstract (fugumt.com page of the same title):
softmax self-attention with key-value caching is what ARL2's fixed-size state replaces.

What the layer computes, per stream b and head h, for latent frame N (0-based) with the
frame's Q, K, V in R^{T x d}:

  out = softmax(scale Q [K_0; ...; K_{N-1}; K]^T) [V_0; ...; V_{N-1}; V]

with K_n, V_n the keys and values of frame n's clean pass; after the clean pass K, V become
K_N, V_N.

Readings taken where the pages leave a step open (each is also listed in the design notes):
  * block-causal: a frame's queries see all earlier frames and every token of their own
    frame (the pages' model is chunkwise causal over frames and bidirectional within one);
  * only clean passes are cached (the pages' clean pass is the one whose context is kept);
    denoising passes attend over the cache plus their own k, v and leave the cache unchanged;
  * scale = 1/sqrt(d); no position encoding or projection inside the layer (the caller's).
"""
from __future__ import annotations

import numpy as np


def cached_attention(q: np.ndarray, k_all: np.ndarray, v_all: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one head's queries q [T, d] over keys / values k_all, v_all [L, d]:
    row t is sum_s p_ts v_s with p_t = softmax(scale * q_t . k_s) over all L cached and current
    keys ([TS] 1; [ABS]).  Subtracting the row maximum before exp only avoids overflow."""
    a = (q @ k_all.T) * scale
    a = a - a.max(axis=1, keepdims=True)
    p = np.exp(a)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v_all


class SoftmaxOracle:
    """The retained softmax layer over a stream of frames.  q, k, v: [B, T, H, d] arrays
    (any float dtype, promoted to fp64)."""

    def __init__(self, head_dim: int, scale: float | None = None):
        self.scale = float(scale) if scale else 1.0 / np.sqrt(head_dim)
        self.k_cache: list[np.ndarray] = []  # clean keys of frames 0..N-1, each [B, T, H, d]
        self.v_cache: list[np.ndarray] = []

    @property
    def frame_index(self) -> int:
        return len(self.k_cache)

    def attend(self, q, k, v) -> np.ndarray:
        """Output of a pass of the current frame (block-causal over the cache and k, v)."""
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        k_all = np.concatenate(self.k_cache + [k], axis=1)  # [B, L, H, d], frames in order
        v_all = np.concatenate(self.v_cache + [v], axis=1)
        B, T, H, _ = q.shape
        out = np.empty_like(q)
        for b in range(B):
            for h in range(H):
                out[b, :, h] = cached_attention(q[b, :, h], k_all[b, :, h], v_all[b, :, h], self.scale)
        return out

    def denoise_step(self, q, k, v) -> np.ndarray:
        return self.attend(q, k, v)

    def commit_frame(self, q, k, v, want_output: bool = True):
        out = self.attend(q, k, v) if want_output else None
        self.k_cache.append(np.asarray(k, dtype=np.float64))
        self.v_cache.append(np.asarray(v, dtype=np.float64))
        return out
