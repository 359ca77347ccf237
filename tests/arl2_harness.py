"""Shared GPU-test harness: runs a seeded stream through libarl2 and through the oracle.

Metrics (the parity bar of the layer):
  output: max |gpu - oracle| / rms(oracle output)  <= 2e-2   (bf16 inputs, fp32 accumulation)
  state:  ||S_gpu - S_oracle||_F / ||S_oracle||_F  <= 1e-3
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from gated_delta_linear_amd import Arl2Layer
from oracle import Arl2Oracle, gate_projections
from synth import make_gate_weights, make_gates, make_hidden, make_pass_inputs, make_phi

OUT_TOL = 2e-2
STATE_TOL = 1e-3


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def dev(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype).contiguous()


def out_err(got: np.ndarray, want: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(np.square(want))))
    return float(np.abs(got - want).max()) / rms


def state_err(got: np.ndarray, want: np.ndarray) -> float:
    n = float(np.linalg.norm(want))
    return float(np.linalg.norm(got - want)) / (n if n > 0 else 1.0)


def make_pair(w, out_dtype=torch.float32):
    phis = make_phi(w)
    layer = Arl2Layer(*[dev(p, torch.bfloat16) for p in phis], batch=w.batch, tokens=w.tokens, out_dtype=out_dtype)
    orc = Arl2Oracle(*[p.astype(np.float64) for p in phis], batch=w.batch)
    return layer, orc


def run_stream(w, check_frames=None, full_output_frames=(), sample_rows=64, out_dtype=torch.float32,
               reuse_denoise=False, frames=None, gated=False):
    """Run `frames` frames of workload w (4-ish denoise passes + 1 clean pass each).

    Outputs are compared on every pass of the frames in `check_frames` (all frames if None):
    in full for frames in `full_output_frames` (or when T is small), otherwise on
    `sample_rows` seeded random token rows.  The state is compared after every frame.
    With reuse_denoise, denoising passes reuse the clean pass's inputs (for long streams,
    where generating unique denoise inputs would dominate; S does not depend on them).
    With gated, the clean pass takes alpha and beta from the gate projections of the frame's
    hidden states (commit_frame_gated; the oracle's gate_projections on the same inputs).
    Returns dict(out_err=max over checks, state_err=list per frame)."""
    frames = w.frames if frames is None else frames
    layer, orc = make_pair(w, out_dtype)
    rng = np.random.default_rng(w.seed + 1000)
    if gated:
        wg, bg = make_gate_weights(w)
        wg_d, bg_d = dev(wg, torch.bfloat16), dev(bg, torch.float32)
    worst_out, state_errs = 0.0, []
    try:
        for f in range(frames):
            check = check_frames is None or f in check_frames
            full = f in full_output_frames or w.tokens * w.heads * w.batch <= 65536
            rows = None if full else np.sort(rng.choice(w.tokens, size=min(sample_rows, w.tokens), replace=False))
            clean = make_pass_inputs(w, f, w.denoise_steps)
            for p in range(w.denoise_steps + 1):
                is_clean = p == w.denoise_steps
                q, k, v = clean if (is_clean or reuse_denoise) else make_pass_inputs(w, f, p)
                qd, kd, vd = (dev(x, torch.bfloat16) for x in (q, k, v))
                if is_clean and gated:
                    x = make_hidden(w, f)
                    beta, alpha = gate_projections(x, wg, bg, w.beta_scale)
                    got = layer.commit_frame_gated(qd, kd, vd, dev(x, torch.bfloat16), wg_d, bg_d, w.beta_scale,
                                                   want_output=check)
                elif is_clean:
                    beta, alpha = make_gates(w, f)
                    got = layer.commit_frame(qd, kd, vd, dev(beta, torch.float32), dev(alpha, torch.float32),
                                             want_output=check)
                else:
                    got = layer.denoise_step(qd, kd, vd)
                if check:
                    got_np = got.double().cpu().numpy()
                    if rows is None:
                        want = orc.query(q, k, v)
                    else:
                        want = orc.query_rows(q, k, v, rows)
                        got_np = got_np[:, rows]
                    worst_out = max(worst_out, out_err(got_np, want))
                if is_clean:
                    orc.state = orc.next_state(k, v, beta, alpha)
                    orc.frame += 1
            s = layer.state().double().cpu().numpy()
            state_errs.append(state_err(s, orc.state))
        assert layer.frame_index == frames
    finally:
        layer.close()
    return {"out_err": worst_out, "state_err": state_errs, "state_norm": float(np.linalg.norm(orc.state))}
