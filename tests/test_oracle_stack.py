"""Pins of the projection and stack oracle (CPU only): the projection against scalar loops and
against permutation weights (which fix the row-vector convention y = x W), the split into parts,
the bf16 rounding against worked ties and a library conversion, and the stack's composition
(the order of Q, K, V in the fused projection, the [B, T, H, d] reading of its output, the layer
kinds) against the layer oracles called directly.  Planted mistakes must each fail a pin.

Sources: "Attend Locally, Remember Linearly" technical summary (gist.science), section 2.1 (the
intra-frame branch reuses the frozen pretrained projections) and section 4 (the 75 % hybrid).
"""
import numpy as np
import pytest
import torch

import oracle.stack_oracle as so
from oracle import Arl2Oracle, SoftmaxOracle

RNG = np.random.default_rng(404)


# --- the projection -------------------------------------------------------------------------

def check_linear_brute_force():
    for (m, k, n) in [(1, 1, 1), (3, 5, 2), (7, 4, 9)]:
        x, w = RNG.standard_normal((m, k)), RNG.standard_normal((k, n))
        y = so.linear(x, w)
        for i in range(m):
            for j in range(n):
                acc = 0.0
                for t in range(k):
                    acc += x[i, t] * w[t, j]
                assert abs(y[i, j] - acc) <= 1e-12, (m, k, n, i, j)


def check_linear_permutation_convention():
    """W with W[pi(j), j] = 1 selects y[:, j] = x[:, pi(j)] (row vectors times W); a transposed
    reading would give x[:, pi^-1(j)], which differs for a permutation that is not its own inverse."""
    k = 6
    pi = np.array([1, 2, 0, 4, 5, 3])
    w = np.zeros((k, k))
    w[pi, np.arange(k)] = 1.0
    x = RNG.standard_normal((5, k))
    np.testing.assert_array_equal(so.linear(x, w), x[:, pi])


def test_linear_brute_force():
    check_linear_brute_force()


def test_linear_row_vector_convention():
    check_linear_permutation_convention()


def test_linear_identity_and_linearity():
    x, x2 = RNG.standard_normal((4, 8)), RNG.standard_normal((4, 8))
    w = RNG.standard_normal((8, 3))
    np.testing.assert_array_equal(so.linear(x, np.eye(8)), x)
    np.testing.assert_allclose(so.linear(2 * x - x2, w), 2 * so.linear(x, w) - so.linear(x2, w), atol=1e-12)


def check_parts():
    x, w = RNG.standard_normal((3, 4)), RNG.standard_normal((4, 12))
    parts = so.linear_parts(x, w, 3)
    assert len(parts) == 3
    full = x @ w
    for p in range(3):
        np.testing.assert_allclose(parts[p], full[:, 4 * p:4 * p + 4], rtol=0, atol=1e-12)


def test_parts_are_consecutive_feature_blocks():
    check_parts()


# --- bf16 rounding --------------------------------------------------------------------------

def check_bf16():
    # worked values: exact, ties to even (down and up), above the tie, sign, a small normal
    cases = {1.0: 1.0, 1 + 2 ** -8: 1.0, 1 + 3 * 2 ** -8: 1 + 2 ** -6, 1 + 2 ** -8 + 2 ** -20: 1 + 2 ** -7,
             -(1 + 3 * 2 ** -8): -(1 + 2 ** -6), 2 ** -100: 2 ** -100, 0.0: 0.0}
    for x, want in cases.items():
        assert so.to_bf16(np.array([x]))[0] == want, x
    # a library conversion on random fp32 values
    x = RNG.standard_normal(4096).astype(np.float32) * 3
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(so.to_bf16(x), lib)


def test_bf16_rounding():
    check_bf16()


# --- the stack ------------------------------------------------------------------------------

def _layers(kinds, H, d, B, T, w_scale=None):
    hd = H * d
    out = []
    for i, kind in enumerate(kinds):
        ly = {"kind": kind,
              "w_qkv": RNG.standard_normal((hd, 3 * hd)) * (w_scale if w_scale is not None else hd ** -0.5),
              "w_o": RNG.standard_normal((hd, hd)) * (w_scale if w_scale is not None else hd ** -0.5)}
        if kind == "arl2":
            ly["phi"] = [np.eye(d)[None] + 0.1 * RNG.standard_normal((H, d, d)) for _ in range(3)]
            betas = [RNG.uniform(0.1, 0.5, (B, T, H)) for _ in range(4)]
            alphas = [RNG.uniform(0.6, 0.95, (B, H)) for _ in range(4)]
            ly["gates"] = (lambda f, b=betas, a=alphas: (b[f], a[f]))
        out.append(ly)
    return out


def check_stack_composition():
    """One ARL2 and one softmax layer with W_qkv = [I | 2 I | 3 I] and W_o = I: the stack equals the
    layer oracles fed q = x, k = 2x, v = 3x, each rounded to bf16 as the stack stores them."""
    B, T, H, d = 2, 5, 2, 4
    hd = H * d
    eye = np.eye(hd)
    for kind in ("arl2", "softmax"):
        ly = _layers([kind], H, d, B, T)[0]
        ly["w_qkv"] = np.concatenate([eye, 2 * eye, 3 * eye], axis=1)
        ly["w_o"] = eye
        stack = so.StackOracle([ly], B, H, d, T)
        ref = Arl2Oracle(*ly["phi"], batch=B) if kind == "arl2" else SoftmaxOracle(d)
        for f in range(2):
            for p in range(2):
                x = so.to_bf16(RNG.standard_normal((B * T, hd)))
                q, k, v = (so.to_bf16(c * x).reshape(B, T, H, d) for c in (1.0, 2.0, 3.0))
                clean = p == 1
                got = stack.run_pass(x, clean)
                if kind == "arl2":
                    want = ref.commit(q, k, v, *ly["gates"](f)) if clean else ref.denoise_step(q, k, v)
                else:
                    want = ref.commit_frame(q, k, v) if clean else ref.denoise_step(q, k, v)
                np.testing.assert_allclose(got, so.to_bf16(want).reshape(B * T, hd), rtol=0, atol=1e-12)


def test_stack_composition():
    check_stack_composition()


def test_stack_of_two_layers_feeds_each_into_the_next():
    """Two layers: the second layer's input is the first one's projected output."""
    B, T, H, d = 1, 6, 2, 4
    layers = _layers(["arl2", "softmax"], H, d, B, T)
    both = so.StackOracle(layers, B, H, d, T)
    first = so.StackOracle(layers[:1], B, H, d, T)
    second = so.StackOracle(layers[1:], B, H, d, T)
    for f in range(2):
        for p in range(2):
            x = so.to_bf16(RNG.standard_normal((B * T, H * d)))
            np.testing.assert_array_equal(both.run_pass(x, p == 1), second.run_pass(first.run_pass(x, p == 1), p == 1))


# --- planted mistakes -------------------------------------------------------------------------

MUTANTS = {
    "projection transposed": ("linear", lambda x, w: np.asarray(x, float) @ np.asarray(w, float).T),
    "parts reversed": ("linear_parts", lambda x, w, parts: np.split(np.asarray(x, float) @ np.asarray(w, float),
                                                                    parts, axis=1)[::-1]),
    "no rounding": ("to_bf16", lambda x: np.asarray(x, dtype=np.float64)),
    "truncation instead of rounding": ("to_bf16", lambda x: (np.ascontiguousarray(np.asarray(x, np.float32))
                                                             .view(np.uint32) & 0xFFFF0000).view(np.float32)
                                                             .astype(np.float64)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(so, attr, fn)
    failed = 0
    for pin in (check_linear_brute_force, check_linear_permutation_convention, check_parts, check_bf16,
                check_stack_composition):
        try:
            pin()
        except (AssertionError, ValueError):
            failed += 1
    assert failed >= 1, name
