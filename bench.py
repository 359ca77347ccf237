"""Throughput of one ARL2 layer on one MI355X: frame-tokens/s at the 1.3B DiT 480p layer shape.

A step is one latent frame of the protocol: 4 denoising passes (query only) + 1 clean pass
(output with S_{N-1}, then the state write), for 1 stream x 12 heads x 1560 tokens x d=128.
Inputs are synthetic (seeded, the shapes and distributions of the workload), pre-staged in
HBM as a ring of 8 unique frames that the timed steps cycle through, so no host work or
PCIe transfer is inside the timed region and the state keeps evolving.

The value is the rate of frames enqueued launch by launch (eager) after W untimed frames;
before those, frames run untimed for --settle seconds (default 1 s), so that the GPU's clocks
have ramped up from idle whatever W is (a fresh GPU runs its first few hundred frames about 12 %
slower).  --graph reports the rate of the same frames replayed from captured HIP graphs instead
(both are in the breakdown).

Prints one JSON line.  Also reports, for the dominant kernel (the fused per-pass kernel),
its average duration inside the workload's frames (an event pair around the four back-to-back
denoising passes of each of 60 frames on the layer's stream, inputs from HBM as in the timed
frames) against the bf16 MFMA peak, and the CPU oracle's rate on a bounded sample.

  python bench.py [--steps K] [--warmup W] [--graph] [--workload dit480p|chunked|long_stream]
  python bench.py --series            per-frame GPU time over the whole stream
  python bench.py --compare-softmax   the retained softmax layer vs the ARL2 layer as its cache grows
  python bench.py --backward          the layer's backward per frame (one pass + the state write)
  python bench.py --stack             a 30-layer attention stack (23 ARL2 + 7 softmax) vs all softmax
  python bench.py --pmc-target        a short run for rocprofv3 counter passes (kernels + a copy)
  python bench.py --summarize-pmc DIR rocprofv3 counter CSVs -> profiles/ traffic summary
  python bench.py --summarize-trace CSV  rocprofv3 kernel trace -> kernel-time table
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "frame-tokens/sec per ARL2 layer at 1560 tok/frame, H=12, d=128; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FWD_KERNEL = "arl2_fwd_kernel"
KERNEL_SOURCES = ["gated_delta_linear_amd/csrc/arl2_fwd.hip", "gated_delta_linear_amd/csrc/arl2_write_partial.h",
                  "gated_delta_linear_amd/csrc/arl2_device.h", "gated_delta_linear_amd/csrc/arl2_kernels.h"]
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "arl2_fwd_dit480p_traffic.json")
RING = 8


def kernel_source_hash() -> str:
    """Hash of the pass kernel's sources with comments, trailing blanks and empty lines removed
    (an edit of a comment leaves the counters taken on the kernel valid)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(line.rstrip() for line in text.splitlines() if line.strip()).encode())
    return h.hexdigest()[:16]


def pass_grid(w) -> int:
    """Work-groups of one denoising-pass launch: one per (stream, head, 128-query tile)."""
    return w.batch * w.heads * ((w.tokens + 127) // 128)


def pass_flops(w) -> float:
    """Algorithmic FLOPs of one pass: per (stream, head) 4 T^2 d (scores and P V) + 2 T d^2
    (the inter-frame read as Q (phi_q S))."""
    T, d = w.tokens, w.head_dim
    return float(w.batch * w.heads * (4 * T * T * d + 2 * T * d * d))


def commit_flops(w) -> float:
    """The state write: per (stream, head) K phi_k, V phi_v, K' S, K'^T (beta R) = 8 T d^2, plus
    2 d^3 for phi_q S."""
    T, d = w.tokens, w.head_dim
    return float(w.batch * w.heads * (8 * T * d * d + 2 * d ** 3))


def frame_flops(w) -> float:
    return (w.denoise_steps + 1) * pass_flops(w) + commit_flops(w)


def state_write_bytes(w) -> float:
    """Algorithmic HBM bytes of the state write alone: per (stream, head) the clean pass's K, V
    (bf16), beta (fp32), S_{N-1} read and S_N written (fp32); per head the maps phi_k, phi_v (bf16)."""
    T, d = w.tokens, w.head_dim
    return float(w.batch * w.heads * (2 * T * d * 2 + 4 * T + 2 * d * d * 4) + w.heads * 2 * d * d * 2)


def frame_distribution(layer, ring, w, out, stream, torch, n=100, backlog=50):
    """Per-frame GPU time of n frames, an event pair around each, enqueued behind a backlog of
    frames (so that the host's pace opens no gaps inside them)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    run_frames(layer, ring, w, backlog, out, stream)
    for f in range(n):
        ev[f][0].record(stream)
        run_frames(layer, ring, w, 1, out, stream, first=f)
        ev[f][1].record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return {"frames": n, "median_us": float(np.median(t)), "p10_us": float(np.percentile(t, 10)),
            "p90_us": float(np.percentile(t, 90)), "min_us": float(t.min()), "max_us": float(t.max())}


def pass_in_frames_us(layer, ring, w, out, stream, torch, n=60, backlog=30):
    """Average duration of the pass kernel inside the frames of the workload: one event pair around
    the denoising passes of each of n frames (back-to-back pass launches, inputs cycling through
    the ring from HBM, as in the timed frames), enqueued behind a backlog of frames; the frame's
    span over its denoise_steps launches.  Returns (mean per launch, per-frame means)."""
    run_frames(layer, ring, w, backlog, out, stream)
    evs = []
    for f in range(n):
        passes, beta, alpha = ring[f % RING]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for p, (q, k, v) in enumerate(passes):
            if p == 0:
                a.record(stream)
            if p < w.denoise_steps:
                if layer.access == "token":
                    layer.denoise_step_seq(q, k, v, beta, out=out, stream=stream)
                else:
                    layer.denoise_step(q, k, v, out=out, stream=stream)
                if p + 1 == w.denoise_steps:
                    b.record(stream)
                    evs.append((a, b))
            elif layer.access == "token":
                layer.commit_frame_seq(q, k, v, beta, alpha, out=out, stream=stream)
            elif alpha is None:
                layer.commit_frame_gated(q, k, v, *beta, out=out, stream=stream)
            else:
                layer.commit_frame(q, k, v, beta, alpha, out=out, stream=stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 / w.denoise_steps for a, b in evs])
    return float(t.mean()), t


def stage_ring(w, torch, gated=False):
    """Device-resident inputs for RING frames: per frame, each pass's q, k, v and the gates
    (beta, alpha), or with gated, the inputs of the gate projections (hidden states x, gate
    weights and biases, beta scale) in place of beta and alpha."""
    from synth import make_gate_weights, make_gates, make_hidden, make_pass_inputs

    dev = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dt)
    if gated:
        wg, bg = make_gate_weights(w)
        wg, bg = dev(wg, torch.bfloat16), dev(bg, torch.float32)
    ring = []
    for f in range(RING):
        passes = [tuple(dev(x, torch.bfloat16) for x in make_pass_inputs(w, f, p)) for p in range(w.denoise_steps + 1)]
        if gated:
            ring.append((passes, (dev(make_hidden(w, f), torch.bfloat16), wg, bg, w.beta_scale), None))
        else:
            beta, alpha = make_gates(w, f)
            ring.append((passes, dev(beta, torch.float32), dev(alpha, torch.float32)))
    torch.cuda.synchronize()
    return ring


def make_layer(w, torch, access="frame"):
    from gated_delta_linear_amd import Arl2Layer
    from synth import make_phi

    phis = [torch.from_numpy(p).to("cuda").to(torch.bfloat16) for p in make_phi(w)]
    return Arl2Layer(*phis, batch=w.batch, tokens=w.tokens, access=access)


def run_frames(layer, ring, w, n, out, stream, first=0):
    """Enqueue n frames of the protocol, frame i using ring slot (first + i) % RING: the
    denoising passes, then the clean pass (output with S_{N-1} and the state write's per-chunk
    sums in one launch, then the write's reduce)."""
    for i in range(n):
        passes, beta, alpha = ring[(first + i) % RING]
        for p, (q, k, v) in enumerate(passes):
            if layer.access == "token":  # the sequential A/B variant: every pass needs beta
                if p < w.denoise_steps:
                    layer.denoise_step_seq(q, k, v, beta, out=out, stream=stream)
                else:
                    layer.commit_frame_seq(q, k, v, beta, alpha, out=out, stream=stream)
            elif p < w.denoise_steps:
                layer.denoise_step(q, k, v, out=out, stream=stream)
            elif alpha is None:  # gated: beta holds (x, w_gates, b_gates, beta_scale)
                layer.commit_frame_gated(q, k, v, *beta, out=out, stream=stream)
            else:
                layer.commit_frame(q, k, v, beta, alpha, out=out, stream=stream)


def capture_frames(layer, ring, w, out, stream, torch):
    """One HIP graph per ring slot, each holding one whole frame (5 pass launches + the
    state write), captured on `stream` (the stream the layer already uses, so no cross-
    stream ordering is recorded).  Replaying graph i % RING for frame i continues the same
    stream of frames (the layer's buffers have fixed addresses)."""
    graphs = []
    for i in range(RING):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            run_frames(layer, ring, w, 1, out, stream, first=i)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def settle_clocks(layer, ring, w, out, stream, torch, seconds):
    """Run untimed frames for about `seconds` of wall time (batches of 50, each synchronised), so
    that the GPU leaves its idle clocks before anything is measured.  Returns the frame count."""
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        run_frames(layer, ring, w, 50, out, stream, first=n)
        torch.cuda.synchronize()
        n += 50
    return n


def time_region(stream, torch, enqueue):
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    enqueue()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end), time.perf_counter() - wall0


def pass_launch_us(layer, ring, w, out, stream, torch, n=40):
    """Average duration of the pass kernel: HIP events around n back-to-back denoising-pass
    launches on the layer's stream (an event pair around every launch would add its own queue
    overhead to each)."""
    def one(i):
        q, k, v = ring[i % RING][0][i % w.denoise_steps]
        if layer.access == "token":
            layer.denoise_step_seq(q, k, v, ring[i % RING][1], out=out, stream=stream)
        else:
            layer.denoise_step(q, k, v, out=out, stream=stream)
    for i in range(4):
        one(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        one(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def commit_launch_us(layer, ring, w, out, stream, torch, pass_out, n=16):
    """Average duration of commit_frame over n back-to-back calls: with the output (the clean
    pass's launch, which also runs the state write's per-chunk work-groups, then the reduce), or
    with out=None (the state write alone).  The calls are enqueued behind n denoising passes, so
    that the device, not the host's per-call cost, sets the pace between the events."""
    def one(i):
        passes, beta, alpha = ring[i % RING]
        q, k, v = passes[-1]
        if layer.access == "token":
            layer.commit_frame_seq(q, k, v, beta, alpha, out=out, want_output=out is not None, stream=stream)
        elif alpha is None:
            layer.commit_frame_gated(q, k, v, *beta, out=out, want_output=out is not None, stream=stream)
        elif out is None:
            layer.commit_frame(q, k, v, beta, alpha, want_output=False, stream=stream)
        else:
            layer.commit_frame(q, k, v, beta, alpha, out=out, stream=stream)
    one(0)
    for i in range(n):
        q, k, v = ring[i % RING][0][i % w.denoise_steps]
        if layer.access == "token":
            layer.denoise_step_seq(q, k, v, ring[i % RING][1], out=pass_out, stream=stream)
        else:
            layer.denoise_step(q, k, v, out=pass_out, stream=stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        one(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def load_traffic(workload: str):
    """HBM bytes per launch of the pass kernel from committed counter passes, if they were
    taken on the current kernel source and on this workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash() or not str(t.get("workload", "")).startswith(workload):
        return None
    return t


def gemm_reference_tflops(torch, n=8192, reps=10) -> float:
    """A measured dense bf16 MFMA reference on the same GPU: torch.matmul (hipBLASLt) of two
    contiguous n x n bf16 matrices, after a warm-up, with HIP events around reps products."""
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12


def probe_ceiling(iters: int = 10000):
    """The chip's sustained dense bf16 MFMA rate from the probe built beside the library (independent
    MFMA chains only; one work-group per CU on 156 and on 256 CUs): {grid: {tflops, clock_ghz}}, or
    None when the probe has not been built."""
    import subprocess

    from gated_delta_linear_amd.build import PROBE_PATH

    if not os.path.exists(PROBE_PATH):
        return None
    res = subprocess.run([PROBE_PATH, str(iters)], capture_output=True, text=True)
    if res.returncode != 0:
        return None
    out = {}
    for line in res.stdout.splitlines():
        r = json.loads(line)
        out[str(r["work_groups"])] = {"tflops": r["tflops"], "clock_ghz": r["clock_ghz"]}
    return out


def cpu_env():
    """BLAS threads the oracle uses, the BLAS build and the CPU model."""
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max((i.get("num_threads", 1) for i in pools), default=1)
        if pools:
            blas = f"{pools[0].get('internal_api', '?')} {pools[0].get('version', '?')}"
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu_model)
    except OSError:  # pragma: no cover
        pass
    return int(threads), blas, cpu_model


def _cpu_line(value, unit, sample, **extra):
    threads, blas, cpu_model = cpu_env()
    line = {"value": value, "unit": unit, "cores": threads, "kind": "oracle", "cpu_model": cpu_model, "blas": blas,
            "sample": sample}
    line.update(extra)
    return line


def cpu_baseline(w, budget_s: float, gated: bool = False, access: str = "frame"):
    """The oracle (numpy fp64) on the first frames of the same stream, in full: every pass's
    output and the state write, until the time budget is spent (at least one frame).  gated:
    beta, alpha from the oracle's gate projections of the hidden states; access "token": the
    token-level (sequential) oracle."""
    from oracle import Arl2Oracle, Arl2SeqOracle, gate_projections
    from synth import make_gate_weights, make_gates, make_hidden, make_pass_inputs, make_phi

    phis = [p.astype(np.float64) for p in make_phi(w)]
    orc = Arl2SeqOracle(*phis, batch=w.batch) if access == "token" else Arl2Oracle(*phis, batch=w.batch)
    if gated:
        wg, bg = make_gate_weights(w)
    frames, busy = 0, 0.0
    while frames < w.frames and (frames == 0 or busy < budget_s):
        inputs = [make_pass_inputs(w, frames, p) for p in range(w.denoise_steps + 1)]
        hidden = make_hidden(w, frames) if gated else None
        beta, alpha = (None, None) if gated else make_gates(w, frames)
        t0 = time.perf_counter()
        if gated:
            beta, alpha = gate_projections(hidden.astype(np.float64), wg.astype(np.float64), bg.astype(np.float64),
                                           w.beta_scale)
        for p, (q, k, v) in enumerate(inputs):
            if access == "token":
                if p < w.denoise_steps:
                    orc.denoise_step(q, k, v, beta)
                else:
                    orc.commit(q, k, v, beta, alpha)
            elif p < w.denoise_steps:
                orc.denoise_step(q, k, v)
            else:
                orc.commit(q, k, v, beta, alpha)
        busy += time.perf_counter() - t0
        frames += 1
    what = ("token-level oracle" if access == "token" else "oracle") + (", gates from the hidden states" if gated else "")
    return _cpu_line(w.batch * w.tokens * frames / busy, "frame-tokens/s",
                     f"{w.name} frames 0..{frames - 1} in full ({w.denoise_steps} denoising passes + clean pass + "
                     f"state write each; {what}), numpy fp64, {busy:.1f} s of CPU work, input generation excluded")


def cpu_baseline_recurrence(w, budget_s: float):
    """The oracle's state recurrence alone (the state write of every frame, no outputs) over the
    stream, its clean passes cycling through RING staged frames as on the GPU, until the stream
    ends or the time budget is spent."""
    from oracle import Arl2Oracle
    from synth import make_gates, make_pass_inputs, make_phi

    orc = Arl2Oracle(*[p.astype(np.float64) for p in make_phi(w)], batch=w.batch)
    ring = []
    for f in range(RING):
        _, k, v = make_pass_inputs(w, f, w.denoise_steps)
        ring.append((k, v) + tuple(make_gates(w, f)))
    frames, busy = 0, 0.0
    while frames < w.frames and (frames == 0 or busy < budget_s):
        k, v, beta, alpha = ring[frames % RING]
        t0 = time.perf_counter()
        orc.commit(None, k, v, beta, alpha, want_output=False)
        busy += time.perf_counter() - t0
        frames += 1
    return _cpu_line(frames / busy, "state writes/s",
                     f"{w.name}: the oracle's state recurrence alone, frames 0..{frames - 1} of {w.frames} (clean passes "
                     f"of {RING} staged frames, cycled), numpy fp64, {busy:.1f} s of CPU work",
                     ms_per_state_write=busy / frames * 1e3)


def cpu_baseline_softmax(w, budget_s: float):
    """The retained softmax layer's oracle over the first frames of the stream, in full (every
    pass attends over the cached clean frames and its own), until the time budget is spent."""
    from oracle import SoftmaxOracle
    from synth import make_pass_inputs

    orc = SoftmaxOracle(w.head_dim)
    frames, busy, per_frame = 0, 0.0, []
    while frames < w.frames and (frames == 0 or busy < budget_s):
        inputs = [make_pass_inputs(w, frames, p) for p in range(w.denoise_steps + 1)]
        t0 = time.perf_counter()
        for p, (q, k, v) in enumerate(inputs):
            if p < w.denoise_steps:
                orc.denoise_step(q, k, v)
            else:
                orc.commit_frame(q, k, v)
        dt = time.perf_counter() - t0
        busy += dt
        per_frame.append(dt * 1e3)
        frames += 1
    return _cpu_line(w.batch * w.tokens * frames / busy, "frame-tokens/s",
                     f"{w.name}: the softmax layer's oracle, frames 0..{frames - 1} in full (frame N attends over N "
                     f"cached frames + its own), numpy fp64, {busy:.1f} s of CPU work, input generation excluded",
                     ms_per_frame=per_frame)


def cpu_baseline_backward(w, budget_s: float):
    """The backward oracle on frames of the same ring as the GPU backward: per frame the clean
    pass's backward (pass_backward) and the state write's (write_backward), with S_{N-1} from the
    oracle's recurrence, until the time budget is spent."""
    from oracle import pass_backward, write_backward
    from oracle.bwd_oracle import forward_states
    from synth import make_gates, make_out_grad, make_pass_inputs, make_phi, make_state_grad

    phi_q, phi_k, phi_v = (p.astype(np.float64) for p in make_phi(w))
    ring = []
    for f in range(RING):
        beta, alpha = make_gates(w, f)
        ring.append({"passes": [make_pass_inputs(w, f, w.denoise_steps)], "beta": beta, "alpha": alpha})
    d = w.head_dim
    states = forward_states(phi_k, phi_v, ring, np.zeros((w.batch, w.heads, d, d)))
    g = make_state_grad(w).astype(np.float64)
    scale = 1.0 / np.sqrt(d)
    frames, busy = 0, 0.0
    while frames == 0 or (busy < budget_s and frames < RING):
        n = RING - 1 - frames  # frames walked in reverse
        (q, k, v), fr = ring[n]["passes"][0], ring[n]
        d_o = make_out_grad(w, n, w.denoise_steps)
        t0 = time.perf_counter()
        pass_backward(q, k, v, d_o, states[n], phi_q, scale)
        write_backward(k, v, fr["beta"], fr["alpha"], states[n], g, phi_k, phi_v)
        busy += time.perf_counter() - t0
        frames += 1
    return _cpu_line(w.batch * w.tokens * frames / busy, "frame-tokens/s",
                     f"{w.name}: the backward oracle, {frames} frame(s) (the clean pass's backward + the state "
                     f"write's), numpy fp64, {busy:.1f} s of CPU work, input generation excluded")


def bench(args):
    import torch

    from synth import WORKLOADS

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU (MI355X)")
    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(stream):
        layer = make_layer(w, torch, access=args.access)
        ring = stage_ring(w, torch, gated=args.gated)
        out = layer.new_output()
        settle_frames = settle_clocks(layer, ring, w, out, stream, torch, args.settle)
        run_frames(layer, ring, w, args.warmup, out, stream)
        torch.cuda.synchronize()

        # eager: every launch enqueued from Python, timed over exactly `steps` frames
        eager_ms, eager_wall = time_region(stream, torch, lambda: run_frames(layer, ring, w, args.steps, out, stream))

        # graphs: the same frames replayed from captured HIP graphs (no host work per launch)
        graphs = capture_frames(layer, ring, w, out, stream, torch)
        for i in range(RING):
            graphs[i].replay()
        torch.cuda.synchronize()
        graph_ms, graph_wall = time_region(stream, torch, lambda: [graphs[i % RING].replay() for i in range(args.steps)])

        # kernel timing: events around each launch, outside the two timed regions above
        pass_us, pass_all = pass_in_frames_us(layer, ring, w, out, stream, torch)
        pass_b2b_us = pass_launch_us(layer, ring, w, out, stream, torch)
        write_us = commit_launch_us(layer, ring, w, None, stream, torch, out)
        clean_us = commit_launch_us(layer, ring, w, out, stream, torch, out)
        dist = frame_distribution(layer, ring, w, out, stream, torch)
        torch.cuda.synchronize()
        device_bytes = layer.device_bytes
        layer.close()
        ceiling = probe_ceiling()  # before the GEMM, which heats the GPU
        gemm_tflops = gemm_reference_tflops(torch)  # last: a long GEMM heats the GPU

    use_graph = args.graph
    elapsed_ms = graph_ms if use_graph else eager_ms
    ms_per_step = elapsed_ms / args.steps
    value = w.batch * w.tokens * args.steps / (elapsed_ms / 1e3)
    achieved = pass_flops(w) / (pass_us * 1e-6) / 1e12
    traffic = load_traffic(w.name)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "frame-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": {"seconds": args.settle, "frames": settle_frames,
                         "note": "untimed frames before the warm-up, until the GPU clocks have ramped up"},
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.batch} stream(s) x {w.heads} heads x {w.tokens} tokens/frame, d={w.head_dim}, "
                        f"{w.denoise_steps} denoising passes + 1 clean pass with state write per frame"
                        + (" (alpha, beta from the gate projections of the hidden states)" if args.gated else "")
                        + (" [token-level access: the sequential A/B variant]" if args.access == "token" else ""),
            "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim, "tokens_per_frame": w.tokens,
            "denoise_steps": w.denoise_steps,
            "beta": (f"{w.beta_scale:.6g} * sigmoid(x . w_beta[h] + b_beta[h]), x ~ N(0,1), w ~ N(0, 1/(H d))"
                     if args.gated else f"sigmoid(N(0,1)) * {w.beta_scale:.6g}"),
            "input_ring_frames": RING, "launch": "hip_graph_per_frame" if use_graph else "eager",
        },
        "roofline": {
            "bound": "mfma", "kernel": FWD_KERNEL, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": traffic["bytes_per_launch"] if traffic else None,
            "flops_per_launch": pass_flops(w), "avg_launch_us": pass_us,
            "measured_reference": {"what": "torch.matmul bf16 8192^3 (hipBLASLt) on the same GPU",
                                   "tflops": gemm_tflops, "frac": achieved / gemm_tflops},
            # what the chip sustains with nothing but MFMAs on the pass's grid (its clock drops
            # below the 2.4 GHz of the nominal peak when every CU is busy)
            "sustained_mfma_ceiling": None if ceiling is None else {
                "what": "bench.py --mfma-ceiling probe: independent bf16 MFMA chains, one work-group per CU",
                "by_work_groups": ceiling, "pass_work_groups": pass_grid(w),
                "frac_of_ceiling": achieved / ceiling["156" if pass_grid(w) <= 156 else "256"]["tflops"]},
        },
        "breakdown": {
            "pass_us": pass_us, "pass_us_p10_p90": [float(np.percentile(pass_all, 10)), float(np.percentile(pass_all, 90))],
            "pass_us_back_to_back": pass_b2b_us,
            "clean_pass_with_write_us": clean_us, "state_write_alone_us": write_us,
            "state_write_alone_GBps": state_write_bytes(w) / (write_us * 1e-6) / 1e9,
            "state_write_alone_hbm_frac": state_write_bytes(w) / (write_us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
            "per_frame_us": dist,
            "frame_us_graph": graph_ms / args.steps * 1e3, "frame_us_eager": eager_ms / args.steps * 1e3,
            "host_wall_s_graph": graph_wall, "host_wall_s_eager": eager_wall,
            "frame_mfma_frac": frame_flops(w) / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "device_bytes": device_bytes,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, gated=args.gated, access=args.access)
    print(json.dumps(line), flush=True)


def series(args):
    """Per-frame GPU time and device memory over a whole stream (the constant-cost check): W
    frames of a throwaway layer are enqueued first (the GPU's clock settles over the first few
    hundred, and they leave a backlog, so that the host's own pace, about the GPU's, does not
    open gaps inside the timed frames), then a fresh layer's frames back to back, an event pair
    around each and no host synchronisation in between; free device memory is read before and
    after the stream."""
    import torch

    from synth import WORKLOADS

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(stream):
        ring = stage_ring(w, torch)
        warm = make_layer(w, torch)
        layer = make_layer(w, torch)
        out = warm.new_output()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(w.frames)]
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        run_frames(warm, ring, w, args.warmup, out, stream)
        free_at = {}
        for f in range(w.frames):
            ev[f][0].record(stream)
            run_frames(layer, ring, w, 1, out, stream, first=f)
            ev[f][1].record(stream)
            if f + 1 in (1, 21, 115, 231):  # allocations happen on the host, at enqueue time
                free_at[str(f + 1)] = torch.cuda.mem_get_info()[0]
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        times = [a.elapsed_time(b) * 1e3 for a, b in ev]
        dev_bytes = layer.device_bytes
        layer.close()
        warm.close()
    t = np.array(times)
    slope = float(np.polyfit(np.arange(len(t)), t, 1)[0]) if len(t) > 2 else 0.0
    at = {str(n): times[n - 1] for n in (1, 2, 21, 115, 231) if n <= len(times)}
    print(json.dumps({"workload": w.name, "frames": w.frames, "warmup_frames": args.warmup,
                      "mean_us": float(t.mean()), "median_us": float(np.median(t)),
                      "p10_us": float(np.percentile(t, 10)), "p90_us": float(np.percentile(t, 90)),
                      "min_us": float(t.min()), "max_us": float(t.max()), "frame_us_at": at,
                      "slope_us_per_100_frames": slope * 100,
                      "slope_pct_of_mean_per_100_frames": slope * 100 / float(t.mean()) * 100,
                      "free_mem_before": int(free0), "free_mem_after_frame": free_at, "free_mem_after": int(free1),
                      "device_bytes": dev_bytes,
                      "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_recurrence(w, args.cpu_budget)}),
          flush=True)


def compare_softmax(args):
    """The retained softmax layer (block-causal attention over its growing K/V cache) against
    the ARL2 layer at the same shape: time per frame (4 denoising passes + clean pass, both
    enqueued launch by launch) and device memory, with N = 0, 20 and 230 frames already cached
    (frames 1, 21 and 231 of a stream), after the same GPU warm-up as the main bench.  Also
    the attention kernel's MFMA rate at the longest cache."""
    import torch

    from gated_delta_linear_amd import SoftmaxLayer
    from synth import WORKLOADS

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()  # default priority
    timed = 4  # frames timed at each cache length
    res = {"metric": "per-layer frame time and memory, retained softmax layer vs ARL2 layer", "workload":
           f"{w.name}: {w.batch} x {w.heads} heads x {w.tokens} tokens/frame, d={w.head_dim}, "
           f"{w.denoise_steps} denoising passes + clean pass per frame", "points": []}
    with torch.cuda.stream(stream):
        ring = stage_ring(w, torch)
        layer = make_layer(w, torch)
        out = layer.new_output()
        run_frames(layer, ring, w, args.warmup, out, stream)
        arl2_ms, _ = time_region(stream, torch, lambda: run_frames(layer, ring, w, 100, out, stream))
        arl2_us = arl2_ms / 100 * 1e3
        arl2_bytes = layer.device_bytes
        layer.close()
        res["arl2"] = {"frame_us": arl2_us, "device_bytes": arl2_bytes}
        for n_cached in (0, 20, 230):
            sm = SoftmaxLayer(w.batch, w.heads, w.head_dim, w.tokens, n_cached + timed)
            for f in range(n_cached):  # fill the cache: clean passes without output
                q, k, v = ring[f % RING][0][-1]
                sm.commit_frame(q, k, v, want_output=False, stream=stream)

            def frames():
                for f in range(timed):
                    passes = ring[(n_cached + f) % RING][0]
                    for p, (q, k, v) in enumerate(passes):
                        if p < w.denoise_steps:
                            sm.denoise_step(q, k, v, out=out, stream=stream)
                        else:
                            sm.commit_frame(q, k, v, out=out, stream=stream)
            ms, _ = time_region(stream, torch, frames)
            frame_us = ms / timed * 1e3
            # frame n_cached + f attends over (n_cached + f + 1) frames of keys; report the mean
            point = {"frames_cached": n_cached, "frame_index_first_timed": n_cached + 1,
                     "frame_us": frame_us, "vs_arl2_time": frame_us / arl2_us,
                     "cache_bytes_after": (n_cached + timed) * 2 * w.batch * w.tokens * w.heads * w.head_dim * 2,
                     "vs_arl2_memory": (n_cached + timed) * 2 * w.batch * w.tokens * w.heads * w.head_dim * 2 / arl2_bytes}
            if n_cached == 230:
                sm.reset()
                for f in range(n_cached):
                    q, k, v = ring[f % RING][0][-1]
                    sm.commit_frame(q, k, v, want_output=False, stream=stream)
                q, k, v = ring[0][0][0]
                n = 10

                def passes():
                    for _ in range(n):
                        sm.denoise_step(q, k, v, out=out, stream=stream)
                pass_ms, _ = time_region(stream, torch, passes)
                keys = (n_cached + 1) * w.tokens
                flops = 4.0 * w.batch * w.heads * w.tokens * keys * w.head_dim
                point["attention_pass_us"] = pass_ms / n * 1e3
                point["attention_tflops"] = flops / (pass_ms / n * 1e-3) / 1e12
                point["attention_mfma_frac"] = point["attention_tflops"] / PEAK_BF16_TFLOPS
            res["points"].append(point)
            sm.close()
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_softmax(w, args.cpu_budget)
    print(json.dumps(res), flush=True)


STACK_LAYERS = 30
STACK_SOFTMAX = (2, 6, 10, 14, 18, 22, 26)  # the 7 of 30 layers kept as softmax attention (every 4th)


def stack_bench(args):
    """The pages' 75 % hybrid stack, attention layers only: 30 attention layers of the workload's
    shape, 23 ARL2 + 7 retained softmax layers (indices STACK_SOFTMAX), each fed by its own fused
    Q, K, V projection of the previous layer's output and followed by its output projection (the
    library's arl2_linear; seeded random-init bf16 weights ~ N(0, 1/(H d)), query rows x 0.5 and
    output weights x 2; no norms, MLPs or residuals), every ARL2 layer with its own maps and gates, against the same stack with all 30
    layers softmax.  Only library kernels run in the timed frames.  Per-frame time (4 denoising
    passes + the clean pass through all 30 layers, launches enqueued back to back; 4 frames timed
    after warm-up) at frames 1, 21 and 231: the softmax caches are pre-filled with 0, 20 and 230
    clean frames of keys and values projected from a random frame (timing does not depend on the
    cached values).  Also the layers' device memory, and the projections alone."""
    import torch

    from gated_delta_linear_amd import Arl2Layer, SoftmaxLayer
    from gated_delta_linear_amd.arl2 import linear
    from gated_delta_linear_amd.stack import AttentionStack
    from synth import WORKLOADS, make_gates, make_phi

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()  # default priority
    B, T, H, d = w.batch, w.tokens, w.heads, w.head_dim
    hd = H * d
    gen = torch.Generator(device="cuda").manual_seed(w.seed + 4242)
    timed, cached = 4, (0, 20, 230)
    max_frames = max(cached) + timed + 24
    with torch.cuda.stream(stream):
        def rnd(*shape, scale=1.0):
            return (torch.randn(*shape, device="cuda", generator=gen) * scale).to(torch.bfloat16)

        def per_layer(i):  # each ARL2 layer's own maps and gates (seeded per layer)
            lw = w.with_(seed=w.seed * 1000 + i)
            phis = [torch.from_numpy(p).to("cuda").to(torch.bfloat16) for p in make_phi(lw)]
            gates = [tuple(torch.from_numpy(g).to("cuda") for g in make_gates(lw, f)) for f in range(RING)]
            return phis, gates

        def qkv_weights():  # query rows x 0.5 and output weights x 2 keep the random stack's activations O(1)
            wqkv = torch.randn(3 * hd, hd, device="cuda", generator=gen) * hd ** -0.5
            wqkv[:hd] *= 0.5
            return wqkv.to(torch.bfloat16)

        weights = [(qkv_weights(), rnd(hd, hd, scale=2 * hd ** -0.5)) for _ in range(STACK_LAYERS)]
        own = {i: per_layer(i) for i in range(STACK_LAYERS) if i not in STACK_SOFTMAX}
        x_in = [rnd(B * T, hd) for _ in range(w.denoise_steps + 1)]  # the stack's input per pass

        def build(hybrid):
            layers = []
            for i, (wqkv, wo) in enumerate(weights):
                kind = "arl2" if hybrid and i not in STACK_SOFTMAX else "softmax"
                ly = {"kind": kind, "w_qkv_t": wqkv, "w_o_t": wo}
                if kind == "arl2":
                    ly["phi"] = own[i][0]
                layers.append(ly)
            return AttentionStack(layers, B, H, d, T, max_frames, stream=stream)

        stacks = {True: build(True), False: build(False)}
        weight_bytes = STACK_LAYERS * 4 * hd * hd * 2
        frame_no = {True: 0, False: 0}

        def frame(hybrid):
            st = stacks[hybrid]
            f = frame_no[hybrid]
            for p in range(w.denoise_steps + 1):
                st.run_pass(x_in[p], p == w.denoise_steps, gates=lambda i: own[i][1][f % RING])
            frame_no[hybrid] += 1

        # cache pre-fill: keys and values projected from a random frame, committed n times
        kv = [torch.empty(B, T, H, d, dtype=torch.bfloat16, device="cuda") for _ in range(3)]

        def prefill(hybrid, n):
            st = stacks[hybrid]
            for i, att in enumerate(st.attn):
                if isinstance(att, SoftmaxLayer):
                    att.reset()
                    linear(x_in[0], weights[i][0], parts=3, out=[t.view(B * T, hd) for t in kv], stream=stream)
                    for _ in range(n):
                        att.commit_frame(None, kv[1], kv[2], want_output=False, stream=stream)

        def projections_only():
            o = stacks[True].o.view(B * T, hd)
            y = stacks[True].x[0]
            for p in range(w.denoise_steps + 1):
                for i in range(STACK_LAYERS):
                    linear(x_in[p], weights[i][0], parts=3, out=[t.view(B * T, hd) for t in kv], stream=stream)
                    linear(o, weights[i][1], out=[y], stream=stream)

        for hybrid in (True, False):
            prefill(hybrid, 0)
            for _ in range(8):  # warm-up (the clock settles; every layer's frame count stays small)
                frame(hybrid)
        points = []
        for n in cached:
            pt = {"frames_cached": n, "frame_index": n + 1}
            for hybrid in (True, False):
                prefill(hybrid, n)
                torch.cuda.synchronize()
                ms, _ = time_region(stream, torch, lambda: [frame(hybrid) for _ in range(timed)])
                key = "hybrid" if hybrid else "all_softmax"
                pt[key + "_ms_per_frame"] = ms / timed
                n_soft = len(STACK_SOFTMAX) if hybrid else STACK_LAYERS
                cache = 2 * (n + timed) * B * T * H * d * 2  # K and V of one softmax layer after the timed frames
                arl2_bytes = next((a.device_bytes for a in stacks[True].attn if isinstance(a, Arl2Layer)), 0)
                pt[key + "_layer_bytes"] = n_soft * cache + (STACK_LAYERS - n_soft) * arl2_bytes
            pt["speedup"] = pt["all_softmax_ms_per_frame"] / pt["hybrid_ms_per_frame"]
            pt["memory_reduction"] = 1 - pt["hybrid_layer_bytes"] / pt["all_softmax_layer_bytes"]
            points.append(pt)
        proj_ms, _ = time_region(stream, torch, lambda: [projections_only() for _ in range(timed)])
        for st in stacks.values():
            st.close()
    # per-frame time grows linearly with the cache; the average over a stream of F = 231 frames
    F = 231
    avg = {}
    for key in ("hybrid", "all_softmax"):
        xs = [p["frames_cached"] for p in points]
        ys = [p[key + "_ms_per_frame"] for p in points]
        slope, icpt = np.polyfit(xs, ys, 1)
        avg[key] = float(icpt + slope * (F - 1) / 2)
    res = {"metric": "per-frame time and memory of a 30-layer attention stack: 23 ARL2 + 7 softmax layers vs all softmax",
           "workload": f"{w.name}: {B} x {H} heads x {T} tokens/frame, d={d}, {w.denoise_steps} denoising passes + clean "
                       f"pass per frame; softmax layers {list(STACK_SOFTMAX)}; fused Q/K/V and output projections "
                       f"(arl2_linear) of random-init bf16 weights; own maps and gates per ARL2 layer; no norms, MLPs "
                       f"or residuals",
           "points": points, "projections_ms_per_frame": proj_ms / timed, "weight_bytes": weight_bytes,
           "stream_average_ms_per_frame": avg, "stream_frames": F,
           "stream_average_speedup": avg["all_softmax"] / avg["hybrid"]}
    print(json.dumps(res), flush=True)


def backward_flops(w) -> float:
    """Algorithmic FLOPs of the backward of one frame (one pass with an output gradient + the state
    write), per (stream, head): the softmax branch's dV, dP, dQ, dK (8 T^2 d); the inter-frame
    read's dO S^T, (.) phi_q^T and Q^T dO (6 T d^2); the state write's per-token products (K phi_k,
    V phi_v, K' S, K' G, R G^T, dR S^T, dR phi_v^T, dU phi_k^T: 16 T d^2) and token sums (K'^T dR,
    V^T dR, K^T dU: 6 T d^2)."""
    T, d = w.tokens, w.head_dim
    return float(w.batch * w.heads * (8 * T * T * d + 28 * T * d * d))


def backward_bench(args):
    """The layer's backward at the workload's shape: one frame = arl2_bwd_pass (the clean pass's
    output gradient) + arl2_bwd_commit, frames cycling through a ring of RING staged frames (the
    forward states S_{N-1} from the GPU forward itself), after W untimed frames.  Also the pass
    and the commit timed alone (HIP events around n back-to-back calls)."""
    import torch

    from gated_delta_linear_amd import Arl2Backward
    from synth import WORKLOADS, make_out_grad, make_phi, make_state_grad

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()  # default priority
    dev = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dt)
    with torch.cuda.stream(stream):
        ring = stage_ring(w, torch)
        layer = make_layer(w, torch)
        states = []
        for f in range(RING):  # S_{N-1} of ring frame f: the state before its commit
            states.append(layer.state(stream=stream))
            run_frames(layer, ring, w, 1, layer.new_output(), stream, first=f)
        layer.close()
        d_outs = [dev(make_out_grad(w, f, w.denoise_steps), torch.float32) for f in range(RING)]
        bw = Arl2Backward(*[dev(p, torch.bfloat16) for p in make_phi(w)], batch=w.batch, tokens=w.tokens, stream=stream)
        bw.begin(dev(make_state_grad(w), torch.float32), stream=stream)
        fs = bw.frame_shape
        dq, dk, dv = (torch.empty(fs, dtype=torch.float32, device="cuda") for _ in range(3))
        dbeta = torch.empty(fs[:3], dtype=torch.float32, device="cuda")
        dalpha = torch.empty((w.batch, w.heads), dtype=torch.float32, device="cuda")

        def one_pass(i):
            (q, k, v), s = ring[i % RING][0][-1], states[i % RING]
            bw.pass_(q, k, v, s, d_outs[i % RING], dq, dk, dv, stream=stream)

        def one_commit(i):
            passes, beta, alpha = ring[i % RING]
            _, k, v = passes[-1]
            bw.commit(k, v, beta, alpha, states[i % RING], dk, dv, dbeta, dalpha, stream=stream)

        def frames(n, first=0):
            for i in range(first, first + n):
                one_pass(RING - 1 - i % RING)  # frames walked in reverse
                one_commit(RING - 1 - i % RING)
        frames(args.warmup)
        ms, wall = time_region(stream, torch, lambda: frames(args.steps))
        n = 20
        pass_ms, _ = time_region(stream, torch, lambda: [one_pass(i) for i in range(n)])
        commit_ms, _ = time_region(stream, torch, lambda: [one_commit(i) for i in range(n)])
        dev_bytes = bw.device_bytes
        bw.close()
    frame_us = ms / args.steps * 1e3
    tokens = w.batch * w.tokens
    line = {
        "metric": "backward frame-tokens/sec per ARL2 layer (one pass with output gradient + state write)",
        "value": tokens / (frame_us * 1e-6), "unit": "frame-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": frame_us / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16/bf16 MFMA, fp32 accumulation", "data": "synthetic",
        "config": {"workload": f"{w.name}: backward, {w.batch} stream(s) x {w.heads} heads x {w.tokens} tokens/frame, "
                               f"d={w.head_dim}, frames walked in reverse", "batch": w.batch, "heads": w.heads,
                   "head_dim": w.head_dim, "tokens_per_frame": w.tokens},
        "breakdown": {"frame_us": frame_us, "pass_us": pass_ms / n * 1e3, "commit_us": commit_ms / n * 1e3,
                      "host_wall_s": wall, "device_bytes": dev_bytes,
                      "algorithmic_gflop_per_frame": backward_flops(w) / 1e9,
                      "frame_tflops": backward_flops(w) / (frame_us * 1e-6) / 1e12,
                      "frame_mfma_frac": backward_flops(w) / (frame_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_backward(w, args.cpu_budget),
    }
    print(json.dumps(line), flush=True)


COPY_BYTES = 2**30  # calibration copy: 1 GiB each way, four times the 256 MB last-level cache


def mfma_ceiling():
    """Runs the sustained-MFMA-rate probe (gated_delta_linear_amd/csrc/probe_mfma_rate.hip, built
    by build() into the package directory): independent 32x32x16 bf16 MFMA chains on 156 and on
    256 work-groups, one per CU; one JSON line per grid with the rate and the clock the waves saw."""
    import subprocess

    from gated_delta_linear_amd.build import PROBE_PATH

    if not os.path.exists(PROBE_PATH):
        sys.exit(f"{PROBE_PATH} is missing: run __graft_entry__.build() first")
    res = subprocess.run([PROBE_PATH], capture_output=True, text=True)
    sys.stdout.write(res.stdout)
    if res.returncode != 0:
        sys.exit(f"probe failed ({res.returncode}): {res.stderr.strip()}")


def pmc_target(args):
    """A short, fixed run for counter passes: a plain device-to-device copy of known size (the
    calibration of FETCH_SIZE / WRITE_SIZE; before each copy another 1 GiB buffer is written,
    so the source comes from HBM, not the last-level cache), then the denoising passes of two
    frames (launches of the pass kernel without the state write's work-groups)."""
    import torch

    from synth import WORKLOADS

    w = WORKLOADS[args.workload]
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    evict = torch.empty_like(src)
    for _ in range(3):
        evict.fill_(2.0)
        dst.copy_(src)
    torch.cuda.synchronize()
    del evict
    layer = make_layer(w, torch)
    ring = stage_ring(w, torch)
    out = layer.new_output()
    stream = torch.cuda.current_stream()
    for f in range(2):
        for p in range(w.denoise_steps):
            q, k, v = ring[f][0][p]
            layer.denoise_step(q, k, v, out=out, stream=stream)
    torch.cuda.synchronize()
    layer.close()
    print(json.dumps({"copy_bytes_each_way": n * 4, "denoise_passes": 2 * w.denoise_steps,
                      "kernel_source_hash": kernel_source_hash()}))


def summarize_pmc(args):
    """Turn two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) into HBM bytes
    per launch of the pass kernel, each scaled by the counter's reading for the plain copy
    (1 GiB read + 1 GiB written).  Writes the JSON bench.py reads."""
    import csv

    def per_kernel(counter):
        rows = []
        for path in glob.glob(os.path.join(args.summarize_pmc, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:
                        rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return rows

    res = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = per_kernel(counter)
        # the runtime's device-to-device copy kernel; the calibration copies are its three largest
        copy = sorted((v for k, v in rows if "copyBuffer" in k), reverse=True)[:3]
        fwd = [v for k, v in rows if FWD_KERNEL in k]
        if len(copy) < 3 or not fwd:
            sys.exit(f"{counter}: copy kernel or {FWD_KERNEL} not found in {args.summarize_pmc}")
        expect_kib = COPY_BYTES / 1024.0
        factor = float(np.median(copy)) / expect_kib
        res[counter] = {"copy_kib_median": float(np.median(copy)), "scale": factor,
                        "fwd_kib_mean": float(np.mean(fwd)), "fwd_bytes": float(np.mean(fwd)) / factor * 1024,
                        "fwd_dispatches": len(fwd)}
    total = res["FETCH_SIZE"]["fwd_bytes"] + res["WRITE_SIZE"]["fwd_bytes"]
    out = {"kernel": FWD_KERNEL, "workload": args.workload, "kernel_source_hash": kernel_source_hash(),
           "bytes_per_launch": total, "counters": res}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def summarize_trace(args):
    """A rocprofv3 kernel trace (CSV) of a bench run -> a markdown table of kernel times, with the
    pass kernel's launches told apart: the denoising passes inside the frames (the four launches
    of 160 x 8-wave work-groups that precede a clean-pass launch and its reduce), the clean passes
    (pass and state-write work-groups in one grid), and its other launches (the back-to-back
    timing and the state write alone)."""
    import csv

    rows = []
    with open(args.summarize_trace) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"],
                         int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))))
    rows.sort()
    is_fwd = [FWD_KERNEL in r[2] for r in rows]
    wgs = sorted({r[3] for r, f in zip(rows, is_fwd) if f})
    small = wgs[0] if wgs else 0
    label = [None] * len(rows)
    # frames: four small-grid passes, one larger-grid pass (the clean pass), then the reduce
    i = 0
    while i + 5 < len(rows):
        names = rows[i:i + 6]
        ok = all(is_fwd[i + j] and names[j][3] == small for j in range(4)) and is_fwd[i + 4] and \
            names[4][3] > small and "commit_reduce" in names[5][2]
        if ok:
            for j in range(4):
                label[i + j] = "pass in frame"
            label[i + 4] = "clean pass"
            label[i + 5] = "reduce in frame"
            i += 6
        else:
            i += 1
    groups = {}
    for r, f, lab in zip(rows, is_fwd, label):
        if lab is None:
            lab = ("pass kernel, other launches" if f else
                   "reduce, other launches" if "commit_reduce" in r[2] else r[2][:90])
        groups.setdefault(lab, []).append((r[1] - r[0]) / 1e3)
    total = sum(sum(v) for v in groups.values())
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---|---|---|---|---|")
    for lab, v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| {lab} | {len(v)} | {np.mean(v):.2f} | {np.min(v):.2f} | {np.max(v):.2f} | "
              f"{100 * sum(v) / total:.1f} % |")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=400,
                    help="untimed frames first (the GPU reaches its steady clock after a few hundred)")
    ap.add_argument("--workload", default="dit480p", choices=["dit480p", "long_stream", "chunked"])
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed frames before the warm-up frames (GPU clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="report the HIP-graph replay rate as the value")
    ap.add_argument("--access", default="frame", choices=["frame", "token"],
                    help="token: the sequential (token-level access) variant, for the A/B against the method")
    ap.add_argument("--gated", action="store_true",
                    help="clean passes take alpha and beta from the gate projections of synthetic hidden states")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle CPU work (min one frame)")
    ap.add_argument("--series", action="store_true")
    ap.add_argument("--compare-softmax", action="store_true",
                    help="the retained softmax layer against the ARL2 layer as the K/V cache grows")
    ap.add_argument("--backward", action="store_true", help="the layer's backward (arl2_bwd.h) per frame")
    ap.add_argument("--stack", action="store_true",
                    help="a 30-layer attention stack, 23 ARL2 + 7 softmax layers, against all softmax")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="the chip's sustained dense bf16 MFMA rate (the probe built beside the library)")
    ap.add_argument("--pmc-target", action="store_true")
    ap.add_argument("--summarize-pmc", metavar="DIR")
    ap.add_argument("--summarize-trace", metavar="CSV", help="rocprofv3 kernel trace -> kernel-time table")
    args = ap.parse_args()
    if args.gated and args.access == "token":
        sys.exit("--gated applies to frame-level access only")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        sys.exit("bench.py measures one GPU: this layer runs without sharding or collectives on a "
                 "single MI355X; --gpus must be 1")
    if args.summarize_trace:
        summarize_trace(args)
    elif args.summarize_pmc:
        summarize_pmc(args)
    elif args.mfma_ceiling:
        mfma_ceiling()
    elif args.pmc_target:
        pmc_target(args)
    elif args.series:
        series(args)
    elif args.compare_softmax:
        compare_softmax(args)
    elif args.backward:
        backward_bench(args)
    elif args.stack:
        stack_bench(args)
    else:
        bench(args)


if __name__ == "__main__":
    main()
