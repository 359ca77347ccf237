"""GPU parity on inputs that drive the pass kernel and the state write through their rarely
taken branches, and the fp32 input path of the interface.

* Sharp attention: Q and K scaled by 4 and 8 (powers of two, exact in bf16), so that within a
  wave's key half a later 32-key unit beats the running maximum by more than the kernel's
  rescale slack and the accumulator and row sums are rescaled with a non-zero accumulator.  The
  test first proves on the CPU that most rows reach that branch.
* Keys whose mapped norm is below knorm_eps (zero rows and rows scaled by 2^-30) in the
  clean pass's write.
* Values at +-2^15 (exact in bf16 and in the fp16 that the P V product uses; the interface
  states |v| <= 65504).
* io_dtype ARL2_F32: fp32 q, k, v and maps, rounded to bf16 on the device, give bitwise the
  bf16 path's results on the same rounded values, and match the oracle on the tiny workload.

Bars: max |err| / rms(output) <= 2e-2 and rel-Frobenius(S) <= 1e-3 (the layer's bars).  Frame 0
(S_0 = 0) checks the softmax branch on its own; frame 1 adds the inter-frame read.
Source: "Attend Locally, Remember Linearly" technical summary (gist.science), section 2.1
(intra-frame branch: the pretrained layer's own softmax; the gated update with K' normalised).
"""
import numpy as np
import pytest
import torch

from gated_delta_linear_amd import Arl2Layer, SoftmaxLayer
from oracle import Arl2Oracle, SoftmaxOracle
from synth import WORKLOADS, Workload, make_gates, make_pass_inputs, make_phi, round_bf16
from tests.arl2_harness import OUT_TOL, STATE_TOL, dev, log, out_err, run_stream, state_err

pytestmark = pytest.mark.gpu

RESCALE_SLACK_LOG2 = 8.0  # the pass kernel raises its running max only past this margin
UNIT = 32


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _rng(seed):
    return np.random.default_rng(seed)


def _normal(rng, shape):
    return round_bf16(rng.standard_normal(shape).astype(np.float32))


def rescale_fraction(q, k, scale):
    """Fraction of (row, key half) pairs where a later unit of the half beats the half's first
    unit's max by more than the slack, i.e. where the kernel rescales a non-zero accumulator."""
    T, d = q.shape
    units = (T + UNIT - 1) // UNIT
    u0 = (units + 1) // 2
    a = (q.astype(np.float64) @ k.astype(np.float64).T) * scale / np.log(2.0)  # log2 units
    hits = total = 0
    for lo, hi in ((0, min(T, u0 * UNIT)), (u0 * UNIT, T)):
        if hi - lo <= UNIT:
            continue
        first = a[:, lo:lo + UNIT].max(axis=1)
        rest = a[:, lo + UNIT:hi].max(axis=1)
        hits += int(np.sum(rest > first + RESCALE_SLACK_LOG2))
        total += T
    return hits / max(total, 1)


def run_frames(phis, frames, B, H, T, out_dtype=torch.float32):
    """frames: list of dicts {passes: [(q, k, v)], beta, alpha} (fp32 arrays, bf16 values).
    Returns (list of per-frame max output errors, list of per-frame state errors)."""
    layer = Arl2Layer(*[dev(p, torch.bfloat16) for p in phis], batch=B, tokens=T, out_dtype=out_dtype)
    orc = Arl2Oracle(*[p.astype(np.float64) for p in phis], batch=B)
    outs, states = [], []
    try:
        for fr in frames:
            worst = 0.0
            for i, (q, k, v) in enumerate(fr["passes"]):
                qd, kd, vd = (dev(x, torch.bfloat16) for x in (q, k, v))
                if i + 1 < len(fr["passes"]):
                    got, want = layer.denoise_step(qd, kd, vd), orc.denoise_step(q, k, v)
                else:
                    got = layer.commit_frame(qd, kd, vd, dev(fr["beta"], torch.float32), dev(fr["alpha"], torch.float32))
                    want = orc.commit(q, k, v, fr["beta"], fr["alpha"])
                g = got.double().cpu().numpy()
                assert np.all(np.isfinite(g))
                worst = max(worst, out_err(g, want))
            outs.append(worst)
            states.append(state_err(layer.state().double().cpu().numpy(), orc.state))
    finally:
        layer.close()
    return outs, states


def _gates(rng, B, T, H, d):
    beta = (rng.uniform(0.1, 0.9, (B, T, H)) * min(1.0, d / T)).astype(np.float32)
    alpha = rng.uniform(0.6, 0.95, (B, H)).astype(np.float32)
    return beta, alpha


@pytest.mark.parametrize("T", [129, 700, 1560])
@pytest.mark.parametrize("mult", [4.0, 8.0])
def test_sharp_attention_rescales(T, mult):
    B, H, d = 1, 2, 128
    rng = _rng(int(T * mult))
    w = Workload("sharp", batch=B, heads=H, head_dim=d, tokens=T, frames=2, denoise_steps=1, seed=int(T + mult))
    phis = make_phi(w)
    frames = []
    for f in range(2):
        passes = []
        for p in range(2):
            q, k, v = (_normal(rng, (B, T, H, d)) for _ in range(3))
            passes.append((q * np.float32(mult), k * np.float32(mult), v))
        frames.append({"passes": passes, "beta": _gates(rng, B, T, H, d)[0], "alpha": _gates(rng, B, T, H, d)[1]})
    q0, k0, _ = frames[0]["passes"][0]
    frac = min(rescale_fraction(q0[0, :, h], k0[0, :, h], 1 / np.sqrt(d)) for h in range(H))
    log(f"sharp T={T} x{mult}: rows rescaling after the first unit {frac:.2f}")
    assert frac > 0.2, frac  # the branch under test is taken on a good share of rows
    outs, states = run_frames(phis, frames, B, H, T)
    log(f"sharp T={T} x{mult}: out_err per frame {outs}, state_err {states}")
    assert max(outs) <= OUT_TOL, outs
    assert max(states) <= STATE_TOL, states


@pytest.mark.parametrize("T", [129, 700])
def test_sharp_attention_kv_cache_instance(T):
    """The plain-attention instance of the pass kernel (retained softmax layers) on sharp
    attention over a growing cache."""
    B, H, d, frames = 1, 2, 128, 3
    rng = _rng(T + 5)
    layer = SoftmaxLayer(B, H, d, T, frames)
    orc = SoftmaxOracle(d)
    worst = 0.0
    frac = 1.0
    try:
        for f in range(frames):
            for p in range(2):
                q, k, v = (_normal(rng, (B, T, H, d)) for _ in range(3))
                q, k = q * np.float32(8.0), k * np.float32(8.0)
                qd, kd, vd = (dev(x, torch.bfloat16) for x in (q, k, v))
                if f == 0 and p == 0:
                    frac = min(rescale_fraction(q[0, :, h], k[0, :, h], 1 / np.sqrt(d)) for h in range(H))
                clean = p == 1
                got = layer.commit_frame(qd, kd, vd) if clean else layer.denoise_step(qd, kd, vd)
                want = orc.attend(q, k, v)
                worst = max(worst, out_err(got.double().cpu().numpy(), want))
                if clean:
                    orc.commit_frame(q, k, v, want_output=False)
    finally:
        layer.close()
    log(f"kv-cache sharp T={T}: rescale fraction {frac:.2f}, out_err {worst:.3e}")
    assert frac > 0.2, frac
    assert worst <= OUT_TOL, worst


@pytest.mark.parametrize("T", [129, 700])
def test_keys_below_norm_eps(T):
    """Zero key rows and key rows of norm ~1e-8 (below knorm_eps = 1e-6 after the map) in the
    denoising and clean passes: K' = K phi_k / eps there, and the write stays within the bar."""
    B, H, d = 1, 2, 128
    rng = _rng(T + 11)
    w = Workload("eps", batch=B, heads=H, head_dim=d, tokens=T, frames=2, denoise_steps=1, seed=T + 11)
    phis = make_phi(w)
    frames = []
    for f in range(2):
        passes = []
        for p in range(2):
            q, k, v = (_normal(rng, (B, T, H, d)) for _ in range(3))
            k[:, ::7] = 0.0
            k[:, 3::11] *= np.float32(2.0 ** -30)
            passes.append((q, k, v))
        beta, alpha = _gates(rng, B, T, H, d)
        frames.append({"passes": passes, "beta": beta, "alpha": alpha})
    outs, states = run_frames(phis, frames, B, H, T)
    log(f"small keys T={T}: out_err {outs}, state_err {states}")
    assert max(outs) <= OUT_TOL, outs
    assert max(states) <= STATE_TOL, states


@pytest.mark.parametrize("T", [129, 1560])
def test_values_at_fp16_range(T):
    """V entries at +-2^15 (one in 64), exact in bf16 and fp16: the P V product's conversion of V
    to fp16 is exact there."""
    B, H, d = 1, 2, 128
    rng = _rng(T + 13)
    w = Workload("bigv", batch=B, heads=H, head_dim=d, tokens=T, frames=2, denoise_steps=1, seed=T + 13)
    phis = make_phi(w)
    frames = []
    for f in range(2):
        passes = []
        for p in range(2):
            q, k, v = (_normal(rng, (B, T, H, d)) for _ in range(3))
            mask = rng.random(v.shape) < 1 / 64
            v[mask] = np.float32(2.0 ** 15) * np.sign(rng.standard_normal(int(mask.sum()))).astype(np.float32)
            passes.append((q, k, v))
        beta, alpha = _gates(rng, B, T, H, d)
        frames.append({"passes": passes, "beta": beta, "alpha": alpha})
    outs, states = run_frames(phis, frames, B, H, T)
    log(f"large V T={T}: out_err {outs}, state_err {states}")
    assert max(outs) <= OUT_TOL, outs
    assert max(states) <= STATE_TOL, states


# --- fp32 inputs (io_dtype ARL2_F32) -----------------------------------------------------------

def test_fp32_inputs_tiny_workload():
    """The tiny workload as specified (fp32 draws): the layer takes the fp32 values, the oracle the
    same values rounded to bf16 (the reading of the fp32 configuration)."""
    w = WORKLOADS["tiny"].with_(bf16_inputs=False)
    phis = make_phi(w)
    layer = Arl2Layer(*[dev(p, torch.float32) for p in phis], batch=w.batch, tokens=w.tokens, io_dtype=torch.float32)
    orc = Arl2Oracle(*[round_bf16(p).astype(np.float64) for p in phis], batch=w.batch)
    worst_o, worst_s = 0.0, 0.0
    try:
        for f in range(w.frames):
            for p in range(w.denoise_steps + 1):
                q, k, v = make_pass_inputs(w, f, p)
                assert not np.array_equal(q, round_bf16(q))  # genuinely fp32 values
                qd, kd, vd = (dev(x, torch.float32) for x in (q, k, v))
                qr, kr, vr = (round_bf16(x) for x in (q, k, v))
                if p < w.denoise_steps:
                    got, want = layer.denoise_step(qd, kd, vd), orc.denoise_step(qr, kr, vr)
                else:
                    beta, alpha = make_gates(w, f)
                    got = layer.commit_frame(qd, kd, vd, dev(beta, torch.float32), dev(alpha, torch.float32))
                    want = orc.commit(qr, kr, vr, beta, alpha)
                worst_o = max(worst_o, out_err(got.double().cpu().numpy(), want))
            worst_s = max(worst_s, state_err(layer.state().double().cpu().numpy(), orc.state))
    finally:
        layer.close()
    log(f"tiny fp32 inputs: out_err {worst_o:.3e}, state_err {worst_s:.3e}")
    assert worst_o <= OUT_TOL and worst_s <= STATE_TOL, (worst_o, worst_s)


@pytest.mark.parametrize("B,H,d,T", [(1, 1, 16, 16), (2, 3, 64, 129), (1, 2, 128, 300),
                                     (1, 12, 128, 1560)])  # the last: the 12-head, 1560-token layer
def test_fp32_inputs_equal_bf16_path_bitwise(B, H, d, T):
    """Device rounding of fp32 inputs = the host's round-to-nearest-even: outputs and state equal
    the bf16 layer's, bitwise, over two frames (denoising, clean pass with and without output)."""
    w = Workload("f32eq", batch=B, heads=H, head_dim=d, tokens=T, frames=2, denoise_steps=1, seed=T + d,
                 bf16_inputs=False)
    phis = make_phi(w)
    l32 = Arl2Layer(*[dev(p, torch.float32) for p in phis], batch=B, tokens=T, io_dtype=torch.float32)
    l16 = Arl2Layer(*[dev(round_bf16(p), torch.bfloat16) for p in phis], batch=B, tokens=T)
    try:
        for f in range(2):
            q, k, v = make_pass_inputs(w, f, 0)
            a = l32.denoise_step(*(dev(x, torch.float32) for x in (q, k, v)))
            b = l16.denoise_step(*(dev(round_bf16(x), torch.bfloat16) for x in (q, k, v)))
            assert torch.equal(a, b)
            q, k, v = make_pass_inputs(w, f, 1)
            beta, alpha = make_gates(w, f)
            ga = (dev(beta, torch.float32), dev(alpha, torch.float32))
            a = l32.commit_frame(*(dev(x, torch.float32) for x in (q, k, v)), *ga, want_output=(f == 0))
            b = l16.commit_frame(*(dev(round_bf16(x), torch.bfloat16) for x in (q, k, v)), *ga, want_output=(f == 0))
            if f == 0:
                assert torch.equal(a, b)
            assert torch.equal(l32.state(), l16.state())
    finally:
        l32.close()
        l16.close()
