"""The C interfaces on the CPU: the library loads, exports every function include/arl2.h,
include/arl2_softmax.h and include/arl2_bwd.h declare, and rejects bad arguments before touching
a device.  No kernel runs here."""
import ctypes
import os
import re

import pytest
import torch

import gated_delta_linear_amd.arl2 as A

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(HERE), "include", "arl2.h")
SOFTMAX_HEADER = os.path.join(os.path.dirname(HERE), "include", "arl2_softmax.h")
BWD_HEADER = os.path.join(os.path.dirname(HERE), "include", "arl2_bwd.h")
LINEAR_HEADER = os.path.join(os.path.dirname(HERE), "include", "arl2_linear.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(A.LIB_PATH):
        from gated_delta_linear_amd.build import build_library
        build_library()
    return A.load_library()


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(arl2_[a-z_]+)\s*\(", text))


def test_header_and_binding_agree():
    assert _declared_functions() == set(A.SIGNATURES)
    assert _declared_functions(SOFTMAX_HEADER) == set(A.SOFTMAX_SIGNATURES)
    assert _declared_functions(BWD_HEADER) == set(A.BWD_SIGNATURES)
    assert _declared_functions(LINEAR_HEADER) == set(A.LINEAR_SIGNATURES)


def test_every_declared_symbol_is_exported(lib):
    for name in (_declared_functions() | _declared_functions(SOFTMAX_HEADER) | _declared_functions(BWD_HEADER)
                 | _declared_functions(LINEAR_HEADER)):
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in range(7):
        assert lib.arl2_status_string(st)
    assert lib.arl2_status_string(99) == b"unknown status"


def test_null_layer_queries(lib):
    assert lib.arl2_frame_index(None) == -1
    assert lib.arl2_device_bytes(None) == 0
    assert lib.arl2_destroy(None) == A.ARL2_OK
    assert lib.arl2_denoise_step(None, None, None, None, None, None) == A.ARL2_E_INVALID_ARG
    assert lib.arl2_commit_frame(None, None, None, None, None, None, None, None) == A.ARL2_E_INVALID_ARG
    assert lib.arl2_commit_frame_gated(None, None, None, None, None, None, None, 1.0, None, None) == \
        A.ARL2_E_INVALID_ARG
    assert lib.arl2_denoise_step_seq(None, None, None, None, None, None, None) == A.ARL2_E_INVALID_ARG
    assert lib.arl2_commit_frame_seq(None, None, None, None, None, None, None, None) == A.ARL2_E_INVALID_ARG
    assert lib.arl2_state_read(None, None, None) == A.ARL2_E_INVALID_ARG
    assert lib.arl2_state_write(None, None, 0, None) == A.ARL2_E_INVALID_ARG
    assert b"NULL" in lib.arl2_last_error()


def _cfg(**kw):
    c = dict(batch=1, heads=2, head_dim=128, tokens_per_frame=64, io_dtype=A.ARL2_BF16, out_dtype=A.ARL2_F32,
             softmax_scale=0.0, knorm_eps=0.0, access=A.ARL2_ACCESS_FRAME)
    c.update(kw)
    return A.Arl2Config(**c)


# Aligned but never dereferenced: every case below is rejected by argument checks that run
# before the device is queried.
FAKE = 0x10000


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), A.ARL2_E_INVALID_ARG),
    (dict(heads=0), A.ARL2_E_INVALID_ARG),
    (dict(tokens_per_frame=0), A.ARL2_E_INVALID_ARG),
    (dict(tokens_per_frame=A.ARL2_MAX_TOKENS + 1), A.ARL2_E_INVALID_ARG),
    (dict(head_dim=32), A.ARL2_E_UNSUPPORTED),
    (dict(head_dim=96), A.ARL2_E_UNSUPPORTED),
    (dict(io_dtype=7), A.ARL2_E_INVALID_ARG),
    (dict(out_dtype=7), A.ARL2_E_INVALID_ARG),
    (dict(softmax_scale=-1.0), A.ARL2_E_INVALID_ARG),
    (dict(softmax_scale=float("nan")), A.ARL2_E_INVALID_ARG),
    (dict(knorm_eps=float("inf")), A.ARL2_E_INVALID_ARG),
    (dict(access=2), A.ARL2_E_INVALID_ARG),
    (dict(access=A.ARL2_ACCESS_TOKEN, head_dim=16), A.ARL2_E_UNSUPPORTED),
    # token-level access: a stream's fp32 inter-frame reads reach 2 GiB (bf16 inputs would not)
    (dict(access=A.ARL2_ACCESS_TOKEN, heads=3000, tokens_per_frame=1500), A.ARL2_E_UNSUPPORTED),
    # a stream's frame slice reaches 2 GiB
    (dict(heads=8192, tokens_per_frame=1024), A.ARL2_E_UNSUPPORTED),
    # the pass kernel's grid: ceil(T / 128) x B x H work-groups beyond 2^24
    (dict(batch=65535, heads=64, tokens_per_frame=1024, head_dim=16), A.ARL2_E_UNSUPPORTED),
])
def test_create_rejects_bad_config(lib, kw, status):
    h = ctypes.c_void_p(123)
    assert lib.arl2_layer_create(ctypes.byref(_cfg(**kw)), FAKE, FAKE, FAKE, None, ctypes.byref(h)) == status
    assert not h.value  # set to NULL on failure
    assert lib.arl2_last_error()


def test_create_rejects_bad_pointers(lib):
    h = ctypes.c_void_p()
    assert lib.arl2_layer_create(None, FAKE, FAKE, FAKE, None, ctypes.byref(h)) == A.ARL2_E_INVALID_ARG
    assert lib.arl2_layer_create(ctypes.byref(_cfg()), None, FAKE, FAKE, None, ctypes.byref(h)) == A.ARL2_E_INVALID_ARG
    assert lib.arl2_layer_create(ctypes.byref(_cfg()), FAKE, FAKE + 8, FAKE, None, ctypes.byref(h)) == \
        A.ARL2_E_INVALID_ARG
    assert b"aligned" in lib.arl2_last_error()
    assert lib.arl2_layer_create(ctypes.byref(_cfg()), FAKE, FAKE, FAKE, None, None) == A.ARL2_E_INVALID_ARG


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device path; a GPU is present")
@pytest.mark.parametrize("io_dtype", [A.ARL2_BF16, A.ARL2_F32])
def test_create_without_device_fails_cleanly(lib, io_dtype):
    """Both input dtypes pass every argument check and stop at the device query."""
    h = ctypes.c_void_p()
    cfg = _cfg(io_dtype=io_dtype)
    assert lib.arl2_layer_create(ctypes.byref(cfg), FAKE, FAKE, FAKE, None, ctypes.byref(h)) == A.ARL2_E_NO_DEVICE
    assert not h.value


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        A.load_library(str(tmp_path / "libarl2.so"))


# --- the retained softmax layer (include/arl2_softmax.h) -----------------------------------

def _scfg(**kw):
    c = dict(batch=1, heads=2, head_dim=128, tokens_per_frame=64, max_frames=4, out_dtype=A.ARL2_F32,
             softmax_scale=0.0)
    c.update(kw)
    return A.SoftmaxConfig(**c)


def test_softmax_null_layer_queries(lib):
    assert lib.arl2_softmax_frame_index(None) == -1
    assert lib.arl2_softmax_device_bytes(None) == 0
    assert lib.arl2_softmax_destroy(None) == A.ARL2_OK
    assert lib.arl2_softmax_reset(None) == A.ARL2_E_INVALID_ARG
    assert lib.arl2_softmax_pass(None, None, None, None, None, None) == A.ARL2_E_INVALID_ARG
    assert lib.arl2_softmax_commit(None, None, None, None, None, None) == A.ARL2_E_INVALID_ARG
    assert b"NULL" in lib.arl2_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), A.ARL2_E_INVALID_ARG),
    (dict(heads=70000), A.ARL2_E_INVALID_ARG),
    (dict(tokens_per_frame=0), A.ARL2_E_INVALID_ARG),
    (dict(max_frames=0), A.ARL2_E_INVALID_ARG),
    (dict(head_dim=32), A.ARL2_E_UNSUPPORTED),
    (dict(out_dtype=5), A.ARL2_E_INVALID_ARG),
    (dict(softmax_scale=float("nan")), A.ARL2_E_INVALID_ARG),
    # one stream's cache of K (max_frames x T x H x d bf16) reaches 2 GiB
    (dict(max_frames=1000, tokens_per_frame=1560, heads=12), A.ARL2_E_UNSUPPORTED),
])
def test_softmax_create_rejects_bad_config(lib, kw, status):
    h = ctypes.c_void_p(123)
    assert lib.arl2_softmax_layer_create(ctypes.byref(_scfg(**kw)), None, ctypes.byref(h)) == status
    assert not h.value
    assert lib.arl2_softmax_layer_create(None, None, ctypes.byref(h)) == A.ARL2_E_INVALID_ARG
    assert lib.arl2_softmax_layer_create(ctypes.byref(_scfg()), None, None) == A.ARL2_E_INVALID_ARG


# --- the backward (include/arl2_bwd.h) -------------------------------------------------------

def test_bwd_null_object(lib):
    assert lib.arl2_bwd_device_bytes(None) == 0
    assert lib.arl2_bwd_destroy(None) == A.ARL2_OK
    assert lib.arl2_bwd_begin(None, None, None) == A.ARL2_E_INVALID_ARG
    assert lib.arl2_bwd_pass(None, None, None, None, None, None, None, None, None, None) == A.ARL2_E_INVALID_ARG
    assert lib.arl2_bwd_commit(None, None, None, None, None, None, None, None, None, None, None) == \
        A.ARL2_E_INVALID_ARG
    assert lib.arl2_bwd_read(None, None, None, None, None, None) == A.ARL2_E_INVALID_ARG
    assert b"NULL" in lib.arl2_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), A.ARL2_E_INVALID_ARG),
    (dict(tokens_per_frame=0), A.ARL2_E_INVALID_ARG),
    (dict(head_dim=16), A.ARL2_E_UNSUPPORTED),
    (dict(access=A.ARL2_ACCESS_TOKEN), A.ARL2_E_UNSUPPORTED),
    (dict(io_dtype=A.ARL2_F32), A.ARL2_E_UNSUPPORTED),
    (dict(knorm_eps=-1.0), A.ARL2_E_INVALID_ARG),
])
def test_bwd_create_rejects_bad_config(lib, kw, status):
    c = dict(batch=1, heads=2, head_dim=128, tokens_per_frame=64, io_dtype=A.ARL2_BF16, out_dtype=A.ARL2_F32,
             softmax_scale=0.0, knorm_eps=0.0, access=A.ARL2_ACCESS_FRAME)
    c.update(kw)
    h = ctypes.c_void_p(123)
    assert lib.arl2_bwd_create(ctypes.byref(A.Arl2Config(**c)), None, None, None, None, ctypes.byref(h)) == status
    assert not h.value



# --- the allocation-free clean pass (arl2_commit_frame_noalloc) ---------------------------------

def _noalloc(lib, cfg, ptrs=None):
    p = [FAKE] * 10 if ptrs is None else ptrs
    return lib.arl2_commit_frame_noalloc(ctypes.byref(cfg) if cfg is not None else None, *p, None)


def test_noalloc_rejects_bad_arguments_before_the_device(lib):
    assert _noalloc(lib, None) == A.ARL2_E_INVALID_ARG
    assert _noalloc(lib, _cfg(batch=0)) == A.ARL2_E_INVALID_ARG
    assert _noalloc(lib, _cfg(io_dtype=A.ARL2_F32)) == A.ARL2_E_UNSUPPORTED
    assert _noalloc(lib, _cfg(access=A.ARL2_ACCESS_TOKEN)) == A.ARL2_E_UNSUPPORTED
    for i in range(8):  # phi_q, phi_k, phi_v, state, (q), k, v, beta, alpha
        ptrs = [FAKE] * 10
        ptrs[i if i < 4 else i + 1] = None
        assert _noalloc(lib, _cfg(), ptrs) == A.ARL2_E_INVALID_ARG, i
    ptrs = [FAKE] * 10
    ptrs[4] = None  # q missing while an output is requested
    assert _noalloc(lib, _cfg(), ptrs) == A.ARL2_E_INVALID_ARG
    ptrs = [FAKE] * 10
    ptrs[5] = FAKE + 4
    assert _noalloc(lib, _cfg(), ptrs) == A.ARL2_E_INVALID_ARG
    assert b"aligned" in lib.arl2_last_error()


def test_noalloc_refuses_frames_beyond_its_array(lib):
    # 4 streams x 12 heads x 4680 tokens (d = 128): about 120 MB of per-chunk partial sums
    assert _noalloc(lib, _cfg(batch=4, heads=12, tokens_per_frame=4680)) == A.ARL2_E_UNSUPPORTED
    assert b"scratch" in lib.arl2_last_error()


# --- the projections (include/arl2_linear.h) ------------------------------------------------------

def _lin(lib, m=256, n=384, k=128, parts=1, y_dtype=A.ARL2_BF16, x=FAKE, w=FAKE, ys=None):
    ys = [FAKE] * parts if ys is None else ys
    arr = (ctypes.c_void_p * max(1, len(ys)))(*ys)
    return lib.arl2_linear(x, w, m, n, k, parts, arr, y_dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(m=-1), A.ARL2_E_INVALID_ARG),
    (dict(k=96), A.ARL2_E_UNSUPPORTED),          # k not a multiple of 64
    (dict(k=(1 << 20) + 64), A.ARL2_E_UNSUPPORTED),
    (dict(n=100), A.ARL2_E_UNSUPPORTED),         # n not a multiple of 8
    (dict(parts=0), A.ARL2_E_INVALID_ARG),
    (dict(parts=5), A.ARL2_E_INVALID_ARG),
    (dict(n=24, parts=4), A.ARL2_E_INVALID_ARG),  # n / parts = 6, not a multiple of 4
    (dict(y_dtype=9), A.ARL2_E_INVALID_ARG),
    (dict(x=None), A.ARL2_E_INVALID_ARG),
    (dict(w=FAKE + 8), A.ARL2_E_INVALID_ARG),
    (dict(parts=2, ys=[FAKE, None]), A.ARL2_E_INVALID_ARG),
    (dict(parts=2, ys=[FAKE, FAKE + 4]), A.ARL2_E_INVALID_ARG),
])
def test_linear_rejects_bad_arguments(lib, kw, status):
    assert _lin(lib, **kw) == status
    assert lib.arl2_last_error()
