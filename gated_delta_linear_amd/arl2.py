"""Python binding of libarl2 (include/arl2.h): argument marshalling only.

Every step of the layer runs in the library's HIP kernels; torch supplies device memory and
the current stream.  Importing works without a GPU; using a layer requires the built
library (``python -m gated_delta_linear_amd.build``) and an MI355X (gfx950) device, and
fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, byref, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

import torch

# ARL2_LIBRARY names another build of the same library (the AddressSanitizer build of the host
# code, for the CPU interface tests); by default the in-tree libarl2.so
LIB_PATH = os.environ.get("ARL2_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libarl2.so")

ARL2_OK = 0
ARL2_E_INVALID_ARG = 1
ARL2_E_UNSUPPORTED = 2
ARL2_E_NO_DEVICE = 3
ARL2_E_OUT_OF_MEMORY = 4
ARL2_E_HIP = 5
ARL2_E_PROTOCOL = 6
ARL2_BF16 = 0
ARL2_F32 = 1
ARL2_ACCESS_FRAME = 0
ARL2_ACCESS_TOKEN = 1
ARL2_MAX_TOKENS = 1 << 20

# every function declared in include/arl2.h, with its ctypes signature
SIGNATURES = {
    "arl2_layer_create": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, POINTER(c_void_p)]),
    "arl2_denoise_step": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "arl2_commit_frame": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "arl2_commit_frame_gated": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_float, c_void_p, c_void_p]),
    "arl2_denoise_step_seq": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "arl2_commit_frame_seq": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p]),
    "arl2_commit_frame_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "arl2_destroy": (c_int, [c_void_p]),
    "arl2_state_read": (c_int, [c_void_p, c_void_p, c_void_p]),
    "arl2_state_write": (c_int, [c_void_p, c_void_p, c_int64, c_void_p]),
    "arl2_frame_index": (c_int64, [c_void_p]),
    "arl2_device_bytes": (c_size_t, [c_void_p]),
    "arl2_status_string": (c_char_p, [c_int]),
    "arl2_last_error": (c_char_p, []),
}

# every function declared in include/arl2_softmax.h (the retained softmax layers)
SOFTMAX_SIGNATURES = {
    "arl2_softmax_layer_create": (c_int, [c_void_p, c_void_p, POINTER(c_void_p)]),
    "arl2_softmax_pass": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "arl2_softmax_commit": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "arl2_softmax_reset": (c_int, [c_void_p]),
    "arl2_softmax_destroy": (c_int, [c_void_p]),
    "arl2_softmax_frame_index": (c_int64, [c_void_p]),
    "arl2_softmax_device_bytes": (c_size_t, [c_void_p]),
}

# every function declared in include/arl2_linear.h (the projections around the attention layers)
LINEAR_SIGNATURES = {
    "arl2_linear": (c_int, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, POINTER(c_void_p), c_int32,
                            c_void_p]),
}

# every function declared in include/arl2_bwd.h (the layer's backward)
BWD_SIGNATURES = {
    "arl2_bwd_create": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, POINTER(c_void_p)]),
    "arl2_bwd_begin": (c_int, [c_void_p, c_void_p, c_void_p]),
    "arl2_bwd_pass": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p]),
    "arl2_bwd_commit": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_void_p]),
    "arl2_bwd_read": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "arl2_bwd_destroy": (c_int, [c_void_p]),
    "arl2_bwd_device_bytes": (c_size_t, [c_void_p]),
}


class Arl2Config(Structure):
    _fields_ = [
        ("batch", c_int32),
        ("heads", c_int32),
        ("head_dim", c_int32),
        ("tokens_per_frame", c_int32),
        ("io_dtype", c_int32),
        ("out_dtype", c_int32),
        ("softmax_scale", c_float),
        ("knorm_eps", c_float),
        ("access", c_int32),
    ]


class SoftmaxConfig(Structure):
    _fields_ = [
        ("batch", c_int32),
        ("heads", c_int32),
        ("head_dim", c_int32),
        ("tokens_per_frame", c_int32),
        ("max_frames", c_int32),
        ("out_dtype", c_int32),
        ("softmax_scale", c_float),
    ]


class Arl2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libarl2.so and attach the C signatures; raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gated_delta_linear_amd.build` "
                           "(the ARL2 layer has no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in {**SIGNATURES, **SOFTMAX_SIGNATURES, **BWD_SIGNATURES, **LINEAR_SIGNATURES}.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().arl2_status_string(status).decode()


def last_error() -> str:
    return load_library().arl2_last_error().decode()


def _check(status: int, what: str) -> None:
    if status != ARL2_OK:
        raise Arl2Error(status, f"{what}: {status_string(status)}: {last_error()}")


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev_tensor(x: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple) -> int:
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if x.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {x.dtype}")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(x.shape)}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return x.data_ptr()


class Arl2Layer:
    """One ARL2 layer on the current GPU (see include/arl2.h for the exact semantics).

    phi_q, phi_k, phi_v: [H, d, d] device tensors of io_dtype (copied at creation).  Frame
    tensors q, k, v are io_dtype [B, T, H, d]; beta fp32 [B, T, H]; alpha fp32 [B, H].
    io_dtype is torch.bfloat16 or torch.float32 (rounded to bf16, nearest even, on the device)."""

    def __init__(self, phi_q: torch.Tensor, phi_k: torch.Tensor, phi_v: torch.Tensor, batch: int, tokens: int,
                 out_dtype: torch.dtype = torch.float32, softmax_scale: float = 0.0, knorm_eps: float = 0.0,
                 stream=None, access: str = "frame", io_dtype: torch.dtype = torch.bfloat16):
        self._lib = load_library()
        self._handle = c_void_p()
        if io_dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("io_dtype must be torch.bfloat16 or torch.float32")
        self.io_dtype = io_dtype
        heads, d, _ = phi_q.shape
        for name, t in (("phi_q", phi_q), ("phi_k", phi_k), ("phi_v", phi_v)):
            _dev_tensor(t, name, io_dtype, (heads, d, d))
        if out_dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
        self.batch, self.heads, self.head_dim, self.tokens = int(batch), int(heads), int(d), int(tokens)
        self.out_dtype = out_dtype
        self.device = phi_q.device
        if access not in ("frame", "token"):
            raise ValueError("access must be 'frame' or 'token'")
        self.access = access
        cfg = Arl2Config(self.batch, self.heads, self.head_dim, self.tokens,
                         ARL2_F32 if io_dtype == torch.float32 else ARL2_BF16,
                         ARL2_F32 if out_dtype == torch.float32 else ARL2_BF16, float(softmax_scale), float(knorm_eps),
                         ARL2_ACCESS_FRAME if access == "frame" else ARL2_ACCESS_TOKEN)
        with torch.cuda.device(self.device):
            st = self._lib.arl2_layer_create(byref(cfg), phi_q.data_ptr(), phi_k.data_ptr(), phi_v.data_ptr(),
                                             _stream_handle(stream), byref(self._handle))
        _check(st, "arl2_layer_create")

    # --- shapes -------------------------------------------------------------------------
    @property
    def frame_shape(self) -> tuple:
        return (self.batch, self.tokens, self.heads, self.head_dim)

    @property
    def state_shape(self) -> tuple:
        return (self.batch, self.heads, self.head_dim, self.head_dim)

    def _ptr(self):
        if not self._handle:
            raise Arl2Error(ARL2_E_PROTOCOL, "layer has been closed")
        return self._handle

    def new_output(self) -> torch.Tensor:
        return torch.empty(self.frame_shape, dtype=self.out_dtype, device=self.device)

    # --- the protocol -------------------------------------------------------------------
    def denoise_step(self, q, k, v, out=None, stream=None) -> torch.Tensor:
        out = self.new_output() if out is None else out
        args = [_dev_tensor(x, n, self.io_dtype, self.frame_shape) for x, n in ((q, "q"), (k, "k"), (v, "v"))]
        po = _dev_tensor(out, "out", self.out_dtype, self.frame_shape)
        _check(self._lib.arl2_denoise_step(self._ptr(), *args, po, _stream_handle(stream)), "arl2_denoise_step")
        return out

    def commit_frame(self, q, k, v, beta, alpha, out=None, want_output: bool = True, stream=None):
        B, T, H, _ = self.frame_shape
        pk = _dev_tensor(k, "k", self.io_dtype, self.frame_shape)
        pv = _dev_tensor(v, "v", self.io_dtype, self.frame_shape)
        pb = _dev_tensor(beta, "beta", torch.float32, (B, T, H))
        pa = _dev_tensor(alpha, "alpha", torch.float32, (B, H))
        if want_output or out is not None:
            out = self.new_output() if out is None else out
            pq = _dev_tensor(q, "q", self.io_dtype, self.frame_shape)
            po = _dev_tensor(out, "out", self.out_dtype, self.frame_shape)
        else:
            pq, po = (q.data_ptr() if isinstance(q, torch.Tensor) else None), None
        _check(self._lib.arl2_commit_frame(self._ptr(), pq, pk, pv, pb, pa, po, _stream_handle(stream)),
               "arl2_commit_frame")
        return out

    def commit_frame_gated(self, q, k, v, x, w_gates, b_gates, beta_scale: float = 1.0, out=None,
                           want_output: bool = True, stream=None):
        """The clean pass with alpha and beta from the gate projections of the hidden states x
        (bf16 [B, T, H d]); w_gates bf16 [2H, H d], b_gates fp32 [2H] (see include/arl2.h)."""
        B, T, H, d = self.frame_shape
        pk = _dev_tensor(k, "k", self.io_dtype, self.frame_shape)
        pv = _dev_tensor(v, "v", self.io_dtype, self.frame_shape)
        px = _dev_tensor(x, "x", torch.bfloat16, (B, T, H * d))
        pw = _dev_tensor(w_gates, "w_gates", torch.bfloat16, (2 * H, H * d))
        pb = _dev_tensor(b_gates, "b_gates", torch.float32, (2 * H,))
        if want_output or out is not None:
            out = self.new_output() if out is None else out
            pq = _dev_tensor(q, "q", self.io_dtype, self.frame_shape)
            po = _dev_tensor(out, "out", self.out_dtype, self.frame_shape)
        else:
            pq, po = None, None
        _check(self._lib.arl2_commit_frame_gated(self._ptr(), pq, pk, pv, px, pw, pb, float(beta_scale), po,
                                                 _stream_handle(stream)), "arl2_commit_frame_gated")
        return out

    # --- token-level access (access="token") --------------------------------------------
    def denoise_step_seq(self, q, k, v, beta, out=None, stream=None) -> torch.Tensor:
        B, T, H, _ = self.frame_shape
        out = self.new_output() if out is None else out
        args = [_dev_tensor(x, n, self.io_dtype, self.frame_shape) for x, n in ((q, "q"), (k, "k"), (v, "v"))]
        pb = _dev_tensor(beta, "beta", torch.float32, (B, T, H))
        po = _dev_tensor(out, "out", self.out_dtype, self.frame_shape)
        _check(self._lib.arl2_denoise_step_seq(self._ptr(), *args, pb, po, _stream_handle(stream)),
               "arl2_denoise_step_seq")
        return out

    def commit_frame_seq(self, q, k, v, beta, alpha, out=None, want_output: bool = True, stream=None):
        B, T, H, _ = self.frame_shape
        args = [_dev_tensor(x, n, self.io_dtype, self.frame_shape) for x, n in ((q, "q"), (k, "k"), (v, "v"))]
        pb = _dev_tensor(beta, "beta", torch.float32, (B, T, H))
        pa = _dev_tensor(alpha, "alpha", torch.float32, (B, H))
        po = None
        if want_output or out is not None:
            out = self.new_output() if out is None else out
            po = _dev_tensor(out, "out", self.out_dtype, self.frame_shape)
        _check(self._lib.arl2_commit_frame_seq(self._ptr(), *args, pb, pa, po, _stream_handle(stream)),
               "arl2_commit_frame_seq")
        return out

    # --- checkpoint hooks ---------------------------------------------------------------
    def state(self, out=None, stream=None) -> torch.Tensor:
        dst = torch.empty(self.state_shape, dtype=torch.float32, device=self.device) if out is None else out
        p = _dev_tensor(dst, "out", torch.float32, self.state_shape)
        _check(self._lib.arl2_state_read(self._ptr(), p, _stream_handle(stream)), "arl2_state_read")
        return dst

    def load_state(self, src: torch.Tensor, frame_index: int, stream=None) -> None:
        p = _dev_tensor(src, "state", torch.float32, self.state_shape)
        _check(self._lib.arl2_state_write(self._ptr(), p, int(frame_index), _stream_handle(stream)),
               "arl2_state_write")

    @property
    def frame_index(self) -> int:
        return int(self._lib.arl2_frame_index(self._ptr()))

    @property
    def device_bytes(self) -> int:
        return int(self._lib.arl2_device_bytes(self._ptr()))

    def close(self) -> None:
        if getattr(self, "_handle", None):
            h, self._handle = self._handle, c_void_p()
            _check(self._lib.arl2_destroy(h), "arl2_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def linear(x: torch.Tensor, w_t: torch.Tensor, parts: int = 1, out_dtype: torch.dtype = torch.bfloat16, out=None,
           stream=None):
    """arl2_linear (include/arl2_linear.h): y = x W with x bf16 [M, K] and W given transposed,
    w_t bf16 [N, K]; returns a list of `parts` outputs [M, N / parts] of out_dtype (the N features
    dealt in order), written into `out` (a list of tensors) when given."""
    lib = load_library()
    if x.dim() != 2 or w_t.dim() != 2 or x.shape[1] != w_t.shape[1]:
        raise ValueError("x must be [M, K] and w_t [N, K]")
    M, K = int(x.shape[0]), int(x.shape[1])
    N = int(w_t.shape[0])
    if out_dtype not in (torch.float32, torch.bfloat16) or parts < 1 or N % parts:
        raise ValueError("out_dtype must be float32 or bfloat16 and parts must divide N")
    px = _dev_tensor(x, "x", torch.bfloat16, (M, K))
    pw = _dev_tensor(w_t, "w_t", torch.bfloat16, (N, K))
    if out is None:
        out = [torch.empty((M, N // parts), dtype=out_dtype, device=x.device) for _ in range(parts)]
    if len(out) != parts:
        raise ValueError("out must hold `parts` tensors")
    ptrs = (c_void_p * parts)(*[_dev_tensor(o.view(M, N // parts) if o.is_contiguous() else o, f"out[{i}]", out_dtype,
                                            (M, N // parts)) for i, o in enumerate(out)])
    _check(lib.arl2_linear(px, pw, M, N, K, parts, ptrs, ARL2_F32 if out_dtype == torch.float32 else ARL2_BF16,
                           _stream_handle(stream)), "arl2_linear")
    return out


def commit_frame_noalloc(phi_q, phi_k, phi_v, state, q, k, v, beta, alpha, out=None, softmax_scale: float = 0.0,
                         knorm_eps: float = 0.0, stream=None):
    """arl2_commit_frame_noalloc (include/arl2.h): the clean pass of one frame on the caller's
    state (fp32 [B, H, d, d], updated in place), with no layer object and no device allocation by
    the library.  phi_* bf16 [H, d, d]; q, k, v bf16 [B, T, H, d]; beta fp32 [B, T, H]; alpha fp32
    [B, H]; out fp32 or bf16 [B, T, H, d], or None (state write only)."""
    lib = load_library()
    heads, d, _ = phi_q.shape
    B, T = int(k.shape[0]), int(k.shape[1])
    frame = (B, T, heads, d)
    phis = [_dev_tensor(t, n, torch.bfloat16, (heads, d, d)) for t, n in ((phi_q, "phi_q"), (phi_k, "phi_k"),
                                                                          (phi_v, "phi_v"))]
    ps = _dev_tensor(state, "state", torch.float32, (B, heads, d, d))
    pk = _dev_tensor(k, "k", torch.bfloat16, frame)
    pv = _dev_tensor(v, "v", torch.bfloat16, frame)
    pb = _dev_tensor(beta, "beta", torch.float32, (B, T, heads))
    pa = _dev_tensor(alpha, "alpha", torch.float32, (B, heads))
    pq = po = None
    out_dtype = ARL2_F32
    if out is not None:
        if out.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("out must be float32 or bfloat16")
        out_dtype = ARL2_F32 if out.dtype == torch.float32 else ARL2_BF16
        po = _dev_tensor(out, "out", out.dtype, frame)
        pq = _dev_tensor(q, "q", torch.bfloat16, frame)
    cfg = Arl2Config(B, heads, d, T, ARL2_BF16, out_dtype, float(softmax_scale), float(knorm_eps), ARL2_ACCESS_FRAME)
    _check(lib.arl2_commit_frame_noalloc(byref(cfg), *phis, ps, pq, pk, pv, pb, pa, po, _stream_handle(stream)),
           "arl2_commit_frame_noalloc")
    return out


class SoftmaxLayer:
    """One retained softmax attention layer with its K/V cache on the current GPU (see
    include/arl2_softmax.h): frame N's passes attend over the cached clean K/V of frames
    0..N-1 and their own k, v; commit() caches k, v as frame N.  q, k, v are bf16 [B, T, H, d]."""

    def __init__(self, batch: int, heads: int, head_dim: int, tokens: int, max_frames: int,
                 out_dtype: torch.dtype = torch.float32, softmax_scale: float = 0.0, device=None, stream=None):
        self._lib = load_library()
        self._handle = c_void_p()
        if out_dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
        self.batch, self.heads, self.head_dim, self.tokens = int(batch), int(heads), int(head_dim), int(tokens)
        self.max_frames = int(max_frames)
        self.out_dtype = out_dtype
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        cfg = SoftmaxConfig(self.batch, self.heads, self.head_dim, self.tokens, self.max_frames,
                            ARL2_F32 if out_dtype == torch.float32 else ARL2_BF16, float(softmax_scale))
        with torch.cuda.device(self.device):
            st = self._lib.arl2_softmax_layer_create(byref(cfg), _stream_handle(stream), byref(self._handle))
        _check(st, "arl2_softmax_layer_create")

    @property
    def frame_shape(self) -> tuple:
        return (self.batch, self.tokens, self.heads, self.head_dim)

    def _ptr(self):
        if not self._handle:
            raise Arl2Error(ARL2_E_PROTOCOL, "layer has been closed")
        return self._handle

    def new_output(self) -> torch.Tensor:
        return torch.empty(self.frame_shape, dtype=self.out_dtype, device=self.device)

    def denoise_step(self, q, k, v, out=None, stream=None) -> torch.Tensor:
        out = self.new_output() if out is None else out
        args = [_dev_tensor(x, n, torch.bfloat16, self.frame_shape) for x, n in ((q, "q"), (k, "k"), (v, "v"))]
        po = _dev_tensor(out, "out", self.out_dtype, self.frame_shape)
        _check(self._lib.arl2_softmax_pass(self._ptr(), *args, po, _stream_handle(stream)), "arl2_softmax_pass")
        return out

    def commit_frame(self, q, k, v, out=None, want_output: bool = True, stream=None):
        pk = _dev_tensor(k, "k", torch.bfloat16, self.frame_shape)
        pv = _dev_tensor(v, "v", torch.bfloat16, self.frame_shape)
        if want_output or out is not None:
            out = self.new_output() if out is None else out
            pq = _dev_tensor(q, "q", torch.bfloat16, self.frame_shape)
            po = _dev_tensor(out, "out", self.out_dtype, self.frame_shape)
        else:
            pq, po = None, None
        _check(self._lib.arl2_softmax_commit(self._ptr(), pq, pk, pv, po, _stream_handle(stream)),
               "arl2_softmax_commit")
        return out

    def reset(self) -> None:
        _check(self._lib.arl2_softmax_reset(self._ptr()), "arl2_softmax_reset")

    @property
    def frame_index(self) -> int:
        return int(self._lib.arl2_softmax_frame_index(self._ptr()))

    @property
    def device_bytes(self) -> int:
        return int(self._lib.arl2_softmax_device_bytes(self._ptr()))

    def close(self) -> None:
        if getattr(self, "_handle", None):
            h, self._handle = self._handle, c_void_p()
            _check(self._lib.arl2_softmax_destroy(h), "arl2_softmax_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class Arl2Backward:
    """Backward of an ARL2 layer over a stream of frames, walked in reverse (see
    include/arl2_bwd.h).  phi_q, phi_k, phi_v: bf16 [H, d, d] device tensors (copied).  Per frame
    N = F-1 .. 0: pass() for every pass whose output enters the loss, then commit(); read() gives
    dL/dS_0 and the dphi sums.  Frame tensors as Arl2Layer's; gradients fp32."""

    def __init__(self, phi_q: torch.Tensor, phi_k: torch.Tensor, phi_v: torch.Tensor, batch: int, tokens: int,
                 softmax_scale: float = 0.0, knorm_eps: float = 0.0, stream=None):
        self._lib = load_library()
        self._handle = c_void_p()
        heads, d, _ = phi_q.shape
        for name, t in (("phi_q", phi_q), ("phi_k", phi_k), ("phi_v", phi_v)):
            _dev_tensor(t, name, torch.bfloat16, (heads, d, d))
        self.batch, self.heads, self.head_dim, self.tokens = int(batch), int(heads), int(d), int(tokens)
        self.device = phi_q.device
        cfg = Arl2Config(self.batch, self.heads, self.head_dim, self.tokens, ARL2_BF16, ARL2_F32,
                         float(softmax_scale), float(knorm_eps), ARL2_ACCESS_FRAME)
        with torch.cuda.device(self.device):
            st = self._lib.arl2_bwd_create(byref(cfg), phi_q.data_ptr(), phi_k.data_ptr(), phi_v.data_ptr(),
                                           _stream_handle(stream), byref(self._handle))
        _check(st, "arl2_bwd_create")

    @property
    def frame_shape(self) -> tuple:
        return (self.batch, self.tokens, self.heads, self.head_dim)

    @property
    def state_shape(self) -> tuple:
        return (self.batch, self.heads, self.head_dim, self.head_dim)

    @property
    def map_shape(self) -> tuple:
        return (self.heads, self.head_dim, self.head_dim)

    def _ptr(self):
        if not self._handle:
            raise Arl2Error(ARL2_E_PROTOCOL, "backward object has been closed")
        return self._handle

    def _f32(self, shape):
        return torch.empty(shape, dtype=torch.float32, device=self.device)

    def begin(self, ds_last=None, stream=None) -> None:
        p = None if ds_last is None else _dev_tensor(ds_last, "ds_last", torch.float32, self.state_shape)
        _check(self._lib.arl2_bwd_begin(self._ptr(), p, _stream_handle(stream)), "arl2_bwd_begin")

    def pass_(self, q, k, v, s_prev, d_out, dq=None, dk=None, dv=None, stream=None):
        """Backward of one pass of the current frame: returns (dq, dk, dv)."""
        fs = self.frame_shape
        dq, dk, dv = (self._f32(fs) if x is None else x for x in (dq, dk, dv))
        args = [_dev_tensor(x, n, torch.bfloat16, fs) for x, n in ((q, "q"), (k, "k"), (v, "v"))]
        ps = _dev_tensor(s_prev, "s_prev", torch.float32, self.state_shape)
        pd = _dev_tensor(d_out, "d_out", torch.float32, fs)
        grads = [_dev_tensor(x, n, torch.float32, fs) for x, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
        _check(self._lib.arl2_bwd_pass(self._ptr(), *args, ps, pd, *grads, _stream_handle(stream)), "arl2_bwd_pass")
        return dq, dk, dv

    def commit(self, k, v, beta, alpha, s_prev, dk, dv, dbeta=None, dalpha=None, stream=None):
        """Backward of the current frame's state write: adds to dk, dv; returns (dbeta, dalpha)."""
        B, T, H, d = self.frame_shape
        dbeta = self._f32((B, T, H)) if dbeta is None else dbeta
        dalpha = self._f32((B, H)) if dalpha is None else dalpha
        pk, pv = (_dev_tensor(x, n, torch.bfloat16, self.frame_shape) for x, n in ((k, "k"), (v, "v")))
        pb = _dev_tensor(beta, "beta", torch.float32, (B, T, H))
        pa = _dev_tensor(alpha, "alpha", torch.float32, (B, H))
        ps = _dev_tensor(s_prev, "s_prev", torch.float32, self.state_shape)
        pdk, pdv = (_dev_tensor(x, n, torch.float32, self.frame_shape) for x, n in ((dk, "dk"), (dv, "dv")))
        pdb = _dev_tensor(dbeta, "dbeta", torch.float32, (B, T, H))
        pda = _dev_tensor(dalpha, "dalpha", torch.float32, (B, H))
        _check(self._lib.arl2_bwd_commit(self._ptr(), pk, pv, pb, pa, ps, pdk, pdv, pdb, pda, _stream_handle(stream)),
               "arl2_bwd_commit")
        return dbeta, dalpha

    def read(self, stream=None):
        """(dL/dS at the current frame, dphi_q, dphi_k, dphi_v) as new fp32 tensors."""
        ds = self._f32(self.state_shape)
        dq, dk, dv = (self._f32(self.map_shape) for _ in range(3))
        _check(self._lib.arl2_bwd_read(self._ptr(), ds.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                       _stream_handle(stream)), "arl2_bwd_read")
        return ds, dq, dk, dv

    @property
    def device_bytes(self) -> int:
        return int(self._lib.arl2_bwd_device_bytes(self._ptr()))

    def close(self) -> None:
        if getattr(self, "_handle", None):
            h, self._handle = self._handle, c_void_p()
            _check(self._lib.arl2_bwd_destroy(h), "arl2_bwd_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

