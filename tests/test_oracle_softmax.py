"""Pins of the retained softmax layer's oracle (CPU only), each against something other than the
oracle's own formula: scalar brute force, torch's scaled_dot_product_attention over the whole
sequence with a block-causal mask, the two-part softmax merge identity, invariants of the
cache protocol, and the ARL2 oracle's intra-frame branch.  Planted mistakes (mutants) must
each fail at least one pin.

Sources: "Attend Locally, Remember Linearly" technical summary (gist.science), section 1 (the
key-value cache that grows by one block per generated frame) and section 2 (the layers kept
as softmax attention); the authors' abstract.
"""
import math

import numpy as np
import pytest
import torch

import oracle.softmax_oracle as so
from oracle import softmax_attention

RNG = np.random.default_rng(1234)


def _frames(B, T, H, d, F, rng=RNG, scale_qk=1.0):
    """F frames of (q, k, v) [B, T, H, d] with bf16-representable values."""
    out = []
    for _ in range(F):
        q, k, v = (torch.from_numpy(rng.standard_normal((B, T, H, d)) * s).to(torch.bfloat16).double().numpy()
                   for s in (scale_qk, scale_qk, 1.0))
        out.append((q, k, v))
    return out


def _run_clean(frames, d):
    orc = so.SoftmaxOracle(d)
    return [orc.commit_frame(q, k, v) for q, k, v in frames]


def test_brute_force_scalar_loops():
    B, T, H, d, F = 1, 3, 2, 4, 3
    frames = _frames(B, T, H, d, F)
    got = _run_clean(frames, d)
    scale = 1.0 / math.sqrt(d)
    for n in range(F):
        q = frames[n][0]
        keys = [frames[m][1] for m in range(n + 1)]
        vals = [frames[m][2] for m in range(n + 1)]
        for b in range(B):
            for h in range(H):
                for t in range(T):
                    scores = [scale * sum(q[b, t, h, i] * kf[b, s, h, i] for i in range(d))
                              for kf in keys for s in range(T)]
                    vs = [vf[b, s, h] for vf in vals for s in range(T)]
                    m = max(scores)
                    w = [math.exp(x - m) for x in scores]
                    z = sum(w)
                    ref = sum(wi * vi for wi, vi in zip(w, vs)) / z
                    np.testing.assert_allclose(got[n][b, t, h], ref, rtol=0, atol=1e-12)


def test_whole_sequence_sdpa_with_block_causal_mask():
    """Frame-by-frame with the cache equals one library attention over all F frames at once
    with the block-causal mask (query frame n sees key frames 0..n)."""
    B, T, H, d, F = 2, 5, 3, 8, 4
    frames = _frames(B, T, H, d, F)
    got = np.concatenate(_run_clean(frames, d), axis=1)  # [B, F T, H, d]
    q, k, v = (torch.from_numpy(np.concatenate([f[i] for f in frames], axis=1)).permute(0, 2, 1, 3)
               for i in range(3))  # [B, H, F T, d]
    fr = torch.arange(F * T) // T
    mask = fr[:, None] >= fr[None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_two_part_merge_identity():
    """Attention over [cache; frame] is the log-sum-exp merge of attention over the cache and
    over the frame, each computed by the library routine."""
    B, T, H, d = 1, 6, 2, 8
    f0, f1 = _frames(B, T, H, d, 2)
    orc = so.SoftmaxOracle(d)
    orc.commit_frame(*f0, want_output=False)
    got = orc.denoise_step(*f1)
    scale = 1.0 / math.sqrt(d)
    for h in range(H):
        q = torch.from_numpy(f1[0][0, :, h])
        parts = []
        for kk, vv in ((f0[1], f0[2]), (f1[1], f1[2])):
            k, v = torch.from_numpy(kk[0, :, h]), torch.from_numpy(vv[0, :, h])
            o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None])[0]
            lse = torch.logsumexp(scale * q @ k.T, dim=1)
            parts.append((o, lse))
        (o0, l0), (o1, l1) = parts
        m = torch.maximum(l0, l1)
        w0, w1 = torch.exp(l0 - m), torch.exp(l1 - m)
        ref = (w0[:, None] * o0 + w1[:, None] * o1) / (w0 + w1)[:, None]
        np.testing.assert_allclose(got[0, :, h], ref.numpy(), rtol=0, atol=1e-12)


def test_denoising_passes_leave_the_cache_unchanged():
    B, T, H, d, F = 1, 4, 2, 8, 3
    frames = _frames(B, T, H, d, F)
    noise = _frames(B, T, H, d, 2 * F, rng=np.random.default_rng(9))
    plain = _run_clean(frames, d)
    orc = so.SoftmaxOracle(d)
    noisy = []
    for n, (q, k, v) in enumerate(frames):
        for j in range(2):
            orc.denoise_step(*noise[2 * n + j])
        noisy.append(orc.commit_frame(q, k, v))
    for a, b in zip(plain, noisy):
        np.testing.assert_array_equal(a, b)


def test_cached_tokens_are_an_unordered_set():
    """Permuting an earlier frame's tokens (keys with their values) leaves later outputs
    unchanged; permuting the current frame's queries permutes its outputs."""
    B, T, H, d = 1, 7, 2, 8
    f0, f1 = _frames(B, T, H, d, 2)
    perm = np.random.default_rng(3).permutation(T)
    base = _run_clean([f0, f1], d)
    f0p = (f0[0], f0[1][:, perm], f0[2][:, perm])
    f1p = (f1[0][:, perm], f1[1], f1[2])
    alt = _run_clean([f0p, f1p], d)
    np.testing.assert_allclose(alt[1], base[1][:, perm], rtol=0, atol=1e-12)


def test_first_frame_is_the_intra_frame_branch():
    """With an empty cache the layer is the frame's own bidirectional attention, as the ARL2
    oracle's intra-frame branch computes it."""
    B, T, H, d = 1, 9, 2, 16
    (f,) = _frames(B, T, H, d, 1)
    got = so.SoftmaxOracle(d).denoise_step(*f)
    for h in range(H):
        ref = softmax_attention(f[0][0, :, h], f[1][0, :, h], f[2][0, :, h], 1.0 / math.sqrt(d))
        np.testing.assert_allclose(got[0, :, h], ref, rtol=0, atol=1e-13)


def test_uniform_scores_average_all_cached_values():
    """Zero queries give equal weights: the output is the mean of every cached and current value."""
    B, T, H, d, F = 1, 4, 1, 8, 3
    frames = _frames(B, T, H, d, F)
    frames[-1] = (np.zeros_like(frames[-1][0]), frames[-1][1], frames[-1][2])
    got = _run_clean(frames, d)[-1]
    ref = np.concatenate([f[2] for f in frames], axis=1).mean(axis=1, keepdims=True)
    np.testing.assert_allclose(got, np.broadcast_to(ref, got.shape), rtol=0, atol=1e-12)


# --- planted mistakes ---------------------------------------------------------------------

_Base = so.SoftmaxOracle  # the unmutated class (the pins look the class up in the module)


class _CachesDenoisePasses(_Base):
    def denoise_step(self, q, k, v):
        out = self.attend(q, k, v)
        self.k_cache.append(np.asarray(k, dtype=np.float64))
        self.v_cache.append(np.asarray(v, dtype=np.float64))
        return out


class _ForgetsCurrentFrame(_Base):
    def attend(self, q, k, v):
        if not self.k_cache:
            return super().attend(q, k, v)
        kc, vc = self.k_cache[-1], self.v_cache[-1]
        return _Base.attend(self._without_last(), q, kc, vc)

    def _without_last(self):
        o = _Base.__new__(_Base)
        o.scale, o.k_cache, o.v_cache = self.scale, self.k_cache[:-1], self.v_cache[:-1]
        return o


class _OnlyLastFrame(_Base):
    def attend(self, q, k, v):
        o = _Base.__new__(_Base)
        o.scale, o.k_cache, o.v_cache = self.scale, self.k_cache[-1:], self.v_cache[-1:]
        return _Base.attend(o, q, k, v)


class _ValuesOutOfOrder(_Base):
    def commit_frame(self, q, k, v, want_output=True):
        out = self.attend(q, k, v) if want_output else None
        self.k_cache.append(np.asarray(k, dtype=np.float64))
        self.v_cache.insert(0, np.asarray(v, dtype=np.float64))
        return out


def _pins_with(cls, monkeypatch):
    monkeypatch.setattr(so, "SoftmaxOracle", cls)
    failed = 0
    for pin in (test_whole_sequence_sdpa_with_block_causal_mask, test_two_part_merge_identity,
                test_denoising_passes_leave_the_cache_unchanged, test_uniform_scores_average_all_cached_values,
                test_brute_force_scalar_loops):
        try:
            pin()
        except AssertionError:
            failed += 1
    return failed


@pytest.mark.parametrize("mutant", [_CachesDenoisePasses, _ForgetsCurrentFrame, _OnlyLastFrame, _ValuesOutOfOrder])
def test_pins_catch_mutant(mutant, monkeypatch):
    assert _pins_with(mutant, monkeypatch) >= 1, mutant.__name__
