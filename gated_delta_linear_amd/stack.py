"""A stack of attention layers with their projections, run through libarl2 only.

Each layer: [Q | K | V] = x W_qkv (one arl2_linear call writing the three [B, T, H, d] tensors),
O = an ARL2 layer or a retained softmax layer over (Q, K, V), x' = O W_o (arl2_linear).  No norms,
MLPs, residual connections or biases: the attention part of an autoregressive video DiT whose
layers the ARL2 conversion keeps (softmax, with a K/V cache) or replaces (ARL2, with a fixed-size
state) ("Attend Locally, Remember Linearly", gist.science technical summary, sections 2.1, 2.3
and 4).  Activations are bf16.  This module only orders library calls and owns the buffers;
every operation runs in the library's kernels.
"""
from __future__ import annotations

import torch

from .arl2 import Arl2Layer, SoftmaxLayer, linear


class AttentionStack:
    """layers: list of dicts with "kind" ("arl2" or "softmax"), "w_qkv_t" bf16 [3 H d, H d] and
    "w_o_t" bf16 [H d, H d] (the projections' weights, transposed: row n holds output feature n),
    and for "arl2" layers "phi" (phi_q, phi_k, phi_v bf16 [H, d, d]).  max_frames bounds the
    softmax layers' caches."""

    def __init__(self, layers, batch: int, heads: int, head_dim: int, tokens: int, max_frames: int, stream=None):
        self.B, self.H, self.d, self.T = batch, heads, head_dim, tokens
        self.layers = layers
        self.stream = stream
        self.attn = []
        for ly in layers:
            if ly["kind"] == "arl2":
                self.attn.append(Arl2Layer(*ly["phi"], batch=batch, tokens=tokens, out_dtype=torch.bfloat16,
                                           stream=stream))
            else:
                self.attn.append(SoftmaxLayer(batch, heads, head_dim, tokens, max_frames, out_dtype=torch.bfloat16,
                                              stream=stream))
        dev = layers[0]["w_qkv_t"].device
        shape = (batch, tokens, heads, head_dim)
        self.qkv = [torch.empty(shape, dtype=torch.bfloat16, device=dev) for _ in range(3)]
        self.o = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        self.x = [torch.empty((batch * tokens, heads * head_dim), dtype=torch.bfloat16, device=dev) for _ in range(2)]

    @property
    def hd(self) -> int:
        return self.H * self.d

    def run_pass(self, x: torch.Tensor, clean: bool, gates=None, out: torch.Tensor | None = None) -> torch.Tensor:
        """One pass of the current frame through every layer; x bf16 [B T, H d].  The clean pass
        commits every layer's frame; gates(i) -> (beta, alpha) device tensors of ARL2 layer i.
        Returns the stack's output: `out` (fp32 or bf16 [B T, H d]) if given, else a bf16 buffer
        that the next call overwrites."""
        M, hd = self.B * self.T, self.hd
        cur = x
        for i, (ly, att) in enumerate(zip(self.layers, self.attn)):
            q, k, v = self.qkv
            linear(cur, ly["w_qkv_t"], parts=3, out=[q.view(M, hd), k.view(M, hd), v.view(M, hd)], stream=self.stream)
            if ly["kind"] == "arl2":
                if clean:
                    beta, alpha = gates(i)
                    att.commit_frame(q, k, v, beta, alpha, out=self.o, stream=self.stream)
                else:
                    att.denoise_step(q, k, v, out=self.o, stream=self.stream)
            elif clean:
                att.commit_frame(q, k, v, out=self.o, stream=self.stream)
            else:
                att.denoise_step(q, k, v, out=self.o, stream=self.stream)
            last = i + 1 == len(self.layers)
            nxt = out if (last and out is not None) else self.x[i % 2]
            linear(self.o.view(M, hd), ly["w_o_t"], out=[nxt], out_dtype=nxt.dtype, stream=self.stream)
            cur = nxt
        return cur

    def device_bytes(self) -> int:
        return sum(a.device_bytes for a in self.attn)

    def close(self) -> None:
        for a in self.attn:
            a.close()
        self.attn = []
