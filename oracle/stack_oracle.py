"""Linear projections and the hybrid attention stack: the plain CPU oracle.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this module.  The product library never imports, links or
calls it, and it shares no code, table or constant with the HIP kernels.

numpy float64; inputs are the values the GPU receives.

Sources.  [TS] technical summary "Attend Locally, Remember Linearly" (gist.science): section 2.1
(the intra-frame branch reuses the pretrained layer's frozen projections; the ARL2 layer reads
the same Q, K, V through its per-head maps), section 2.3 and section 4 (the converted 1.3B model
keeps softmax attention in a quarter of its layers and replaces the rest: the 75 % hybrid).
[ABS] the authors' abstract.

A projection is y = x W on token rows (row-vector convention, no bias): x [M, K], W [K, N].  One
attention layer of the stack, for a frame's tokens x [B T, H d]:

  [Q | K | V] = x W_qkv            (W_qkv [H d, 3 H d]; Q, K, V read as [B, T, H, d])
  O = layer(Q, K, V)               (an ARL2 layer or a retained softmax layer, with its own state)
  x' = O W_o                       (W_o [H d, H d])

and the stack applies its layers in order to each pass's input.  Readings (the pages give the
architecture only in words): no norms, MLPs, residual connections or biases (the attention part
of the stack only); the activations between the operations are bf16 tensors, so the oracle
rounds them to bf16 (nearest even) where the stack stores them: after each projection and after
each attention layer.
"""
from __future__ import annotations

import numpy as np

from .arl2_oracle import Arl2Oracle
from .softmax_oracle import SoftmaxOracle


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W: y[m, n] = sum_k x[m, k] W[k, n]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64)


def linear_parts(x: np.ndarray, w: np.ndarray, parts: int) -> list[np.ndarray]:
    """y = x W with its N output features dealt, in order, to `parts` outputs of N / parts each."""
    y = linear(x, w)
    return np.split(y, parts, axis=1)


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even), returned as float64: keep the sign, the
    8-bit exponent and the top 7 mantissa bits of the fp32 value, rounding the dropped 16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


class StackOracle:
    """A stack of attention layers with their projections.  layers: list of dicts with "kind"
    ("arl2" or "softmax"), "w_qkv" [H d, 3 H d], "w_o" [H d, H d] and, for "arl2", "phi" (phi_q,
    phi_k, phi_v [H, d, d]) and "gates" (a function frame -> (beta [B, T, H], alpha [B, H]))."""

    def __init__(self, layers, batch: int, heads: int, head_dim: int, tokens: int):
        self.B, self.H, self.d, self.T = batch, heads, head_dim, tokens
        self.layers = layers
        self.state = []
        for ly in layers:
            if ly["kind"] == "arl2":
                self.state.append(Arl2Oracle(*[np.asarray(p, dtype=np.float64) for p in ly["phi"]], batch=batch))
            else:
                self.state.append(SoftmaxOracle(head_dim))
        self.frame = 0

    def run_pass(self, x: np.ndarray, clean: bool, round_output: bool = True) -> np.ndarray:
        """One pass of the current frame through every layer; x [B T, H d].  The clean pass
        commits every layer's frame (ARL2 state write, softmax cache append).  With round_output
        False the last projection's result is returned unrounded (a stack whose output tensor is
        fp32)."""
        B, T, H, d = self.B, self.T, self.H, self.d
        x = np.asarray(x, dtype=np.float64)
        for i, (ly, st) in enumerate(zip(self.layers, self.state)):
            q, k, v = (to_bf16(p).reshape(B, T, H, d) for p in linear_parts(x, ly["w_qkv"], 3))
            if ly["kind"] == "arl2":
                if clean:
                    beta, alpha = ly["gates"](self.frame)
                    o = st.commit(q, k, v, beta, alpha)
                else:
                    o = st.denoise_step(q, k, v)
            else:
                o = st.commit_frame(q, k, v) if clean else st.denoise_step(q, k, v)
            x = linear(to_bf16(o).reshape(B * T, H * d), ly["w_o"])
            if round_output or i + 1 < len(self.layers):
                x = to_bf16(x)
        if clean:
            self.frame += 1
        return x
