"""ctypes binding of libdora_hip.so (the C ABI declared in include/dora.h).

Argument marshalling only: these functions check that the torch tensors they
are given have the shapes, dtypes and device the C ABI expects, pass their data
pointers and torch's current HIP stream, and raise DoraError on a non-zero
status.  Every step of the computation runs in the HIP kernels; there is no
fallback.  Importing this module raises ImportError when the library has not
been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DORA_HIP_LIB selects another build of the same library (the host-sanitizer
# build of the CPU validation check); by default the in-tree libdora_hip.so.
LIB_PATH = os.environ.get("DORA_HIP_LIB") or os.path.join(_HERE, "libdora_hip.so")

DORA_OK, DORA_INVALID_ARG, DORA_UNSUPPORTED, DORA_HIP_ERROR = 0, 1, 2, 3
DTYPE_CODE = {torch.bfloat16: 0, torch.float16: 1}

EXPORTS = (
    "dora_norm_workspace_bytes",
    "dora_norm_factored",
    "dora_norm_factored_cached",
    "dora_row_sqnorm",
    "dora_compose_fwd",
    "dora_lora_compose_fwd",
    "dora_lora_compose_bwd_workspace_bytes",
    "dora_lora_compose_bwd",
    "dora_compose_bwd_workspace_bytes",
    "dora_compose_bwd",
    "dora_compose_bwd_noalloc",
    "dora_norm_bwd_workspace_bytes",
    "dora_norm_bwd",
    "dora_last_error",
    "dora_version",
)


class DoraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc for gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.dora_norm_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.dora_norm_workspace_bytes.restype = sz
    lib.dora_norm_factored.argtypes = [vp, vp, vp, i64, i64, i64, f32, i32, vp, vp, sz, vp]
    lib.dora_norm_factored.restype = i32
    lib.dora_norm_factored_cached.argtypes = [vp, vp, vp, vp, i64, i64, i64, f32, i32, vp, vp, sz, vp]
    lib.dora_norm_factored_cached.restype = i32
    lib.dora_row_sqnorm.argtypes = [vp, i64, i64, i32, vp, vp]
    lib.dora_row_sqnorm.restype = i32
    lib.dora_compose_fwd.argtypes = [vp, vp, vp, vp, f32, i64, i64, i32, i32, vp, vp]
    lib.dora_compose_fwd.restype = i32
    lib.dora_lora_compose_fwd.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i64, i32, i32, vp, vp]
    lib.dora_lora_compose_fwd.restype = i32
    lib.dora_lora_compose_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.dora_lora_compose_bwd_workspace_bytes.restype = sz
    lib.dora_lora_compose_bwd.argtypes = [vp, vp, vp, vp, vp, vp, f32, i64, i64, i64, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.dora_lora_compose_bwd.restype = i32
    lib.dora_compose_bwd_workspace_bytes.argtypes = [i64, i64]
    lib.dora_compose_bwd_workspace_bytes.restype = sz
    lib.dora_compose_bwd.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.dora_compose_bwd.restype = i32
    lib.dora_compose_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, i32, i32, vp, vp, vp, vp]
    lib.dora_compose_bwd_noalloc.restype = i32
    lib.dora_norm_bwd_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.dora_norm_bwd_workspace_bytes.restype = sz
    lib.dora_norm_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, f32, i32, vp, vp, vp, sz, vp]
    lib.dora_norm_bwd.restype = i32
    lib.dora_last_error.argtypes = []
    lib.dora_last_error.restype = ctypes.c_char_p
    lib.dora_version.argtypes = []
    lib.dora_version.restype = ctypes.c_char_p
    return lib


LIB = _load()


def dora_last_error() -> str:
    return LIB.dora_last_error().decode()


def dora_version() -> str:
    return LIB.dora_version().decode()


def _check(status: int) -> None:
    if status != DORA_OK:
        raise DoraError(status, dora_last_error())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _matrix(t, name, shape, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _code(t) -> int:
    if t.dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported dtype {t.dtype}; bf16 and fp16 are")
    if t.device.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    return DTYPE_CODE[t.dtype]


def dora_norm_workspace_bytes(out: int, in_: int, r: int, dtype=torch.bfloat16) -> int:
    code = DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(LIB.dora_norm_workspace_bytes(out, in_, r, code))


def dora_compose_bwd_workspace_bytes(T: int, out: int) -> int:
    return int(LIB.dora_compose_bwd_workspace_bytes(T, out))


def dora_norm_factored(W0, A, B, s: float, norm_out=None, workspace=None):
    """norm_out[i] = ||W0_i + s B_i A||_2 (fp32) via the factored kernels."""
    code = _code(W0)
    out, in_ = W0.shape
    r = A.shape[0]
    dev = W0.device
    _matrix(W0, "W0", (out, in_), W0.dtype, dev)
    _matrix(A, "A", (r, in_), W0.dtype, dev)
    _matrix(B, "B", (out, r), W0.dtype, dev)
    if norm_out is None:
        norm_out = torch.empty(out, dtype=torch.float32, device=dev)
    _matrix(norm_out, "norm_out", (out,), torch.float32, dev)
    need = dora_norm_workspace_bytes(out, in_, r, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(LIB.dora_norm_factored(_ptr(W0), _ptr(A), _ptr(B), out, in_, r, float(s), code, _ptr(norm_out),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)))
    return norm_out


def dora_norm_factored_cached(W0, A, B, base_sq, s: float, norm_out=None, workspace=None):
    """dora_norm_factored with the base term ||W0_i||^2 taken from base_sq (fp32 [out])."""
    code = _code(W0)
    out, in_ = W0.shape
    r = A.shape[0]
    dev = W0.device
    _matrix(W0, "W0", (out, in_), W0.dtype, dev)
    _matrix(A, "A", (r, in_), W0.dtype, dev)
    _matrix(B, "B", (out, r), W0.dtype, dev)
    _matrix(base_sq, "base_sq", (out,), torch.float32, dev)
    if norm_out is None:
        norm_out = torch.empty(out, dtype=torch.float32, device=dev)
    _matrix(norm_out, "norm_out", (out,), torch.float32, dev)
    need = dora_norm_workspace_bytes(out, in_, r, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(LIB.dora_norm_factored_cached(_ptr(W0), _ptr(A), _ptr(B), _ptr(base_sq), out, in_, r, float(s), code,
                                         _ptr(norm_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(dev)))
    return norm_out


def dora_row_sqnorm(W0, sq_out=None):
    """sq_out[i] = ||W0_i||^2 (fp32)."""
    code = _code(W0)
    out, in_ = W0.shape
    dev = W0.device
    _matrix(W0, "W0", (out, in_), W0.dtype, dev)
    if sq_out is None:
        sq_out = torch.empty(out, dtype=torch.float32, device=dev)
    _matrix(sq_out, "sq_out", (out,), torch.float32, dev)
    _check(LIB.dora_row_sqnorm(_ptr(W0), out, in_, code, _ptr(sq_out), _stream(dev)))
    return sq_out


def dora_compose_fwd(base, lora, mag, norm, s: float, add_base: bool = False, y=None):
    """y = (g-1)*base + g*s*lora (+ base), g = mag/norm per column."""
    code = _code(base)
    T, out = base.shape
    dev = base.device
    _matrix(lora, "lora", (T, out), base.dtype, dev)
    _matrix(mag, "mag", (out,), torch.float32, dev)
    _matrix(norm, "norm", (out,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(base)
    _matrix(y, "y", (T, out), base.dtype, dev)
    _check(LIB.dora_compose_fwd(_ptr(base), _ptr(lora), _ptr(mag), _ptr(norm), float(s), T, out, code,
                                int(bool(add_base)), _ptr(y), _stream(dev)))
    return y


def dora_lora_compose_fwd(base, h, B, mag, norm, s: float, add_base: bool = False, y=None):
    """y = (g-1)*base + g*s*(h B^T) (+ base), g = mag/norm per column; lora never stored."""
    code = _code(base)
    T, out = base.shape
    r = h.shape[1]
    dev = base.device
    _matrix(h, "h", (T, r), base.dtype, dev)
    _matrix(B, "B", (out, r), base.dtype, dev)
    _matrix(mag, "mag", (out,), torch.float32, dev)
    _matrix(norm, "norm", (out,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(base)
    _matrix(y, "y", (T, out), base.dtype, dev)
    _check(LIB.dora_lora_compose_fwd(_ptr(base), _ptr(h), _ptr(B), _ptr(mag), _ptr(norm), float(s), T, out, r, code,
                                     int(bool(add_base)), _ptr(y), _stream(dev)))
    return y


def dora_lora_compose_bwd_workspace_bytes(T: int, out: int, r: int) -> int:
    return int(LIB.dora_lora_compose_bwd_workspace_bytes(T, out, r))


def dora_lora_compose_bwd(dy, base, h, B, mag, norm, s: float, add_base: bool = False, d_base=None, d_B=None,
                          d_mag=None, workspace=None, want_d_base: bool = True):
    """(d_base, d_B, d_mag) of the fused compose; d_base is None if not wanted."""
    code = _code(dy)
    T, out = dy.shape
    r = h.shape[1]
    dev = dy.device
    _matrix(base, "base", (T, out), dy.dtype, dev)
    _matrix(h, "h", (T, r), dy.dtype, dev)
    _matrix(B, "B", (out, r), dy.dtype, dev)
    _matrix(mag, "mag", (out,), torch.float32, dev)
    _matrix(norm, "norm", (out,), torch.float32, dev)
    if d_base is None and want_d_base:
        d_base = torch.empty_like(dy)
    if d_B is None:
        d_B = torch.empty_like(B)
    if d_mag is None:
        d_mag = torch.empty(out, dtype=torch.float32, device=dev)
    if d_base is not None:
        _matrix(d_base, "d_base", (T, out), dy.dtype, dev)
    _matrix(d_B, "d_B", (out, r), dy.dtype, dev)
    _matrix(d_mag, "d_mag", (out,), torch.float32, dev)
    need = dora_lora_compose_bwd_workspace_bytes(T, out, r)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(LIB.dora_lora_compose_bwd(_ptr(dy), _ptr(base), _ptr(h), _ptr(B), _ptr(mag), _ptr(norm), float(s), T, out,
                                     r, code, int(bool(add_base)), _ptr(d_base), _ptr(d_B), _ptr(d_mag),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)))
    return d_base, d_B, d_mag


def dora_compose_bwd(dy, base, lora, mag, norm, s: float, add_base: bool = False, d_lora=None, d_base=None,
                     d_mag=None, workspace=None, want_d_base: bool = True):
    """(d_lora, d_base, d_mag) of the compose; d_base is None if not wanted."""
    code = _code(dy)
    T, out = dy.shape
    dev = dy.device
    _matrix(base, "base", (T, out), dy.dtype, dev)
    _matrix(lora, "lora", (T, out), dy.dtype, dev)
    _matrix(mag, "mag", (out,), torch.float32, dev)
    _matrix(norm, "norm", (out,), torch.float32, dev)
    if d_lora is None:
        d_lora = torch.empty_like(dy)
    if d_base is None and want_d_base:
        d_base = torch.empty_like(dy)
    if d_mag is None:
        d_mag = torch.empty(out, dtype=torch.float32, device=dev)
    _matrix(d_lora, "d_lora", (T, out), dy.dtype, dev)
    if d_base is not None:
        _matrix(d_base, "d_base", (T, out), dy.dtype, dev)
    _matrix(d_mag, "d_mag", (out,), torch.float32, dev)
    need = dora_compose_bwd_workspace_bytes(T, out)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(LIB.dora_compose_bwd(_ptr(dy), _ptr(base), _ptr(lora), _ptr(mag), _ptr(norm), float(s), T, out, code,
                                int(bool(add_base)), _ptr(d_lora), _ptr(d_base), _ptr(d_mag), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(dev)))
    return d_lora, d_base, d_mag


def dora_compose_bwd_noalloc(dy, base, lora, mag, norm, s: float, add_base: bool = False, d_lora=None, d_base=None,
                             d_mag=None, want_d_base: bool = True):
    """dora_compose_bwd with the library's own scratch in place of a workspace
    (the entry point that allocates nothing; outputs passed in are written in
    place, missing ones are allocated here, outside the library call)."""
    code = _code(dy)
    T, out = dy.shape
    dev = dy.device
    _matrix(base, "base", (T, out), dy.dtype, dev)
    _matrix(lora, "lora", (T, out), dy.dtype, dev)
    _matrix(mag, "mag", (out,), torch.float32, dev)
    _matrix(norm, "norm", (out,), torch.float32, dev)
    if d_lora is None:
        d_lora = torch.empty_like(dy)
    if d_base is None and want_d_base:
        d_base = torch.empty_like(dy)
    if d_mag is None:
        d_mag = torch.empty(out, dtype=torch.float32, device=dev)
    _matrix(d_lora, "d_lora", (T, out), dy.dtype, dev)
    if d_base is not None:
        _matrix(d_base, "d_base", (T, out), dy.dtype, dev)
    _matrix(d_mag, "d_mag", (out,), torch.float32, dev)
    _check(LIB.dora_compose_bwd_noalloc(_ptr(dy), _ptr(base), _ptr(lora), _ptr(mag), _ptr(norm), float(s), T, out,
                                        code, int(bool(add_base)), _ptr(d_lora), _ptr(d_base), _ptr(d_mag),
                                        _stream(dev)))
    return d_lora, d_base, d_mag


def dora_norm_bwd_workspace_bytes(out: int, in_: int, r: int, dtype=torch.bfloat16) -> int:
    return int(LIB.dora_norm_bwd_workspace_bytes(out, in_, r, DTYPE_CODE.get(dtype, -1)))


def dora_norm_bwd(W0, A, B, norm, d_norm, s: float, d_A=None, d_B=None, workspace=None):
    """(d_A, d_B): the gradients of sum(d_norm * n) with respect to A and B,
    n = the weight norm of W0 + s B A (norm: the forward's n)."""
    code = _code(W0)
    out, in_ = W0.shape
    r = A.shape[0]
    dev = W0.device
    _matrix(W0, "W0", (out, in_), W0.dtype, dev)
    _matrix(A, "A", (r, in_), W0.dtype, dev)
    _matrix(B, "B", (out, r), W0.dtype, dev)
    _matrix(norm, "norm", (out,), torch.float32, dev)
    _matrix(d_norm, "d_norm", (out,), torch.float32, dev)
    if d_A is None:
        d_A = torch.empty_like(A)
    if d_B is None:
        d_B = torch.empty_like(B)
    _matrix(d_A, "d_A", (r, in_), W0.dtype, dev)
    _matrix(d_B, "d_B", (out, r), W0.dtype, dev)
    need = dora_norm_bwd_workspace_bytes(out, in_, r, W0.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(LIB.dora_norm_bwd(_ptr(W0), _ptr(A), _ptr(B), _ptr(norm), _ptr(d_norm), out, in_, r, float(s), code,
                             _ptr(d_A), _ptr(d_B), _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(dev)))
    return d_A, d_B
