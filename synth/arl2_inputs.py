"""Seeded synthetic inputs for the ARL2 layer workloads.

Every tensor is drawn with numpy's PCG64 from ``SeedSequence(seed, spawn_key=...)`` so a
single (workload, frame, pass, tensor) tuple always yields the same values, whichever
consumer asks for them.  Float draws are fp32; tensors the layer reads in bf16 are rounded
to bf16 with round-to-nearest-even here, so the oracle (which promotes them to fp64) and
the GPU (which receives the bf16 bits) see bit-identical values.

Distributions (one recipe for all workloads):
  Q, K, V           ~ N(0, 1)
  phi_q, phi_k, phi_v = I + N(0, 0.1^2 / d), one d x d map per head, drawn once per layer
  alpha (frame, b, h) = sigmoid(N(2, 0.5))
  beta (frame, b, t, h) = sigmoid(N(0, 1)) * min(1, d / T)   ("eff" mode, the default)
                        = sigmoid(N(0, 1))                    ("literal" mode)
  dL/d out (frame, pass) ~ N(0, 1) fp32;  dL/dS after the last frame ~ N(0, 1 / d) fp32
                        (the backward's incoming gradients)

The min(1, d/T) factor keeps the frame-parallel write contractive when a frame holds far
more tokens than the head dimension; the update formula itself is untouched (beta is an
input of the layer).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

# spawn-key namespaces, so that per-pass draws never collide with per-layer draws
_NS_PASS = 0
_NS_GATE = 1
_NS_PHI = 2
_NS_HIDDEN = 3
_NS_GATE_W = 4
_NS_GRAD = 5

_T_Q, _T_K, _T_V = 0, 1, 2
_T_ALPHA, _T_BETA = 0, 1


@dataclass(frozen=True)
class Workload:
    """Shape and protocol of one synthetic stream of frames."""

    name: str
    batch: int              # B independent streams
    heads: int              # H
    head_dim: int           # d
    tokens: int             # T tokens per frame (or per chunk, in chunked generation)
    frames: int             # latent frames (or chunks) in the stream
    denoise_steps: int      # query-only passes per frame before the clean pass
    seed: int
    beta_mode: str = "eff"  # "eff" or "literal"
    bf16_inputs: bool = True

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def beta_scale(self) -> float:
        if self.beta_mode == "literal":
            return 1.0
        if self.beta_mode == "eff":
            return min(1.0, self.head_dim / self.tokens)
        raise ValueError(f"unknown beta_mode {self.beta_mode!r}")


WORKLOADS = {
    # 1 head, d=16, 4 frames of 16 tokens, 2 denoise steps + 1 clean commit each, seed 0
    "tiny": Workload("tiny", batch=1, heads=1, head_dim=16, tokens=16, frames=4,
                     denoise_steps=2, seed=0),
    # one layer of a 1.3B video DiT at 480p: 12 heads, d=128, 30x52 latent patches per frame
    "dit480p": Workload("dit480p", batch=1, heads=12, head_dim=128, tokens=1560, frames=21,
                        denoise_steps=4, seed=1),
    # the same layer over a long stream (231 latent frames, about 921 video frames)
    "long_stream": Workload("long_stream", batch=1, heads=12, head_dim=128, tokens=1560,
                            frames=231, denoise_steps=4, seed=2),
    # chunked generation: 3 latent frames per chunk handled as one unit, 4 streams
    "chunked": Workload("chunked", batch=4, heads=12, head_dim=128, tokens=4680, frames=77,
                        denoise_steps=4, seed=3),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value in bf16 conversion")
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value (returned as fp32)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def _sigmoid32(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def make_phi(w: Workload) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per-head d x d maps phi_q, phi_k, phi_v as fp32 arrays [H, d, d] (bf16-representable
    when the workload feeds bf16)."""
    d = w.head_dim
    out = []
    for t in range(3):
        noise = _rng(w.seed, _NS_PHI, t).standard_normal((w.heads, d, d), dtype=np.float32)
        phi = np.eye(d, dtype=np.float32)[None] + noise * np.float32(0.1 / np.sqrt(d))
        out.append(round_bf16(phi) if w.bf16_inputs else phi.astype(np.float32))
    return out[0], out[1], out[2]


def make_pass_inputs(w: Workload, frame: int, pass_idx: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V for one pass of one frame, fp32 arrays [B, T, H, d].

    pass_idx 0 .. denoise_steps-1 are the denoising passes, pass_idx == denoise_steps is the
    clean pass whose K, V feed the state write."""
    shape = (w.batch, w.tokens, w.heads, w.head_dim)
    out = []
    for t in (_T_Q, _T_K, _T_V):
        x = _rng(w.seed, _NS_PASS, frame, pass_idx, t).standard_normal(shape, dtype=np.float32)
        out.append(round_bf16(x) if w.bf16_inputs else x)
    return out[0], out[1], out[2]


def make_gates(w: Workload, frame: int) -> tuple[np.ndarray, np.ndarray]:
    """beta fp32 [B, T, H] and alpha fp32 [B, H] for the state write of one frame."""
    a = _rng(w.seed, _NS_GATE, frame, _T_ALPHA).normal(2.0, 0.5, size=(w.batch, w.heads))
    alpha = _sigmoid32(a.astype(np.float32))
    b = _rng(w.seed, _NS_GATE, frame, _T_BETA).standard_normal((w.batch, w.tokens, w.heads),
                                                               dtype=np.float32)
    beta = (_sigmoid32(b) * np.float32(w.beta_scale)).astype(np.float32)
    return beta, alpha


def make_hidden(w: Workload, frame: int) -> np.ndarray:
    """Hidden states x of the clean pass of one frame (the input of the gate projections), fp32
    [B, T, H d] ~ N(0, 1), bf16-representable when the workload feeds bf16."""
    x = _rng(w.seed, _NS_HIDDEN, frame).standard_normal((w.batch, w.tokens, w.heads * w.head_dim),
                                                         dtype=np.float32)
    return round_bf16(x) if w.bf16_inputs else x


def make_gate_weights(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """Random-init gate projection weights fp32 [2H, H d] ~ N(0, 1 / (H d)) (so that a gate's
    logit for N(0, 1) hidden states is about N(0, 1)), bf16-representable, and biases fp32 [2H]:
    0 for the beta rows, 2 for the alpha rows (alpha near sigmoid(2) ~ 0.88, as make_gates)."""
    dm = w.heads * w.head_dim
    wt = _rng(w.seed, _NS_GATE_W, 0).standard_normal((2 * w.heads, dm), dtype=np.float32)
    wt = wt * np.float32(1.0 / np.sqrt(dm))
    bias = np.concatenate([np.zeros(w.heads, np.float32), np.full(w.heads, 2.0, np.float32)])
    return (round_bf16(wt) if w.bf16_inputs else wt), bias


def make_out_grad(w: Workload, frame: int, pass_idx: int) -> np.ndarray:
    """Gradient of a loss with respect to one pass's output, fp32 [B, T, H, d] ~ N(0, 1)."""
    return _rng(w.seed, _NS_GRAD, frame, pass_idx).standard_normal(
        (w.batch, w.tokens, w.heads, w.head_dim), dtype=np.float32)


def make_state_grad(w: Workload) -> np.ndarray:
    """Gradient with respect to the state after the last frame, fp32 [B, H, d, d] ~ N(0, 1 / d)."""
    g = _rng(w.seed, _NS_GRAD, 1 << 20).standard_normal((w.batch, w.heads, w.head_dim, w.head_dim),
                                                      dtype=np.float32)
    return g * np.float32(1.0 / np.sqrt(w.head_dim))

