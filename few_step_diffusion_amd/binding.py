"""Thin ctypes binding of libfsd.so (include/fsd.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libfsd.so.  Tensors must live on the GPU; each call enqueues on torch's
current stream.  The library is loaded on first use and a missing or
unloadable library raises FsdError — there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "FsdError", "library_path", "lib", "abi_version", "lora_merge", "workspace_bytes",
    "lora_down", "lora_up", "lora_linear", "lora_linear_plan", "lora_linear_noalloc", "renoise", "euler_step", "token_embed",
    "token_head", "token_head_euler", "token_embed_mx", "mx_lora_down_mx", "mx_lora_up_q", "mx_lora_linear", "mx_lora_linear_plan",
    "mx_workspace_bytes",
    "mx_quantize", "mx_padded_k", "mx_scale_bytes",
    "mx_scale_offsets", "mx_pack_scales", "mx_unpack_scales", "mx_lora_down", "mx_lora_up",
    "mx_lora_up_swiglu_mx", "attention_workspace_bytes", "attention", "StepGraph",
    "EPI_NONE", "EPI_SWIGLU",
]

EPI_NONE = 0
EPI_SWIGLU = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfsd.so")
_lib = None

_STATUS = {0: "FSD_OK", 1: "FSD_EINVAL", 2: "FSD_EALIGN", 3: "FSD_EUNSUPPORTED",
           4: "FSD_EWORKSPACE", 5: "FSD_EHIP"}


class FsdError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}")


def library_path() -> str:
    return _LIB_PATH


_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_int = ctypes.c_int

_SIGS = {
    "fsd_abi_version": ([], _int),
    "fsd_status_str": ([_int], ctypes.c_char_p),
    "fsd_lora_merge": ([_int, ctypes.POINTER(_c_void_p), ctypes.POINTER(_c_void_p),
                        ctypes.POINTER(_i64), _c_void_p, _i64, _i64, _c_void_p, _c_void_p,
                        _c_void_p], _int),
    "fsd_lora_linear_workspace_bytes": ([_i64, _i64], ctypes.c_size_t),
    "fsd_lora_down": ([_c_void_p, _i64, _c_void_p, _f32, _c_void_p, _i64, _i64, _i64, _i64,
                       _c_void_p], _int),
    "fsd_lora_up": ([_c_void_p, _i64, _c_void_p, _c_void_p, _i64, _c_void_p, _c_void_p,
                     _c_void_p, _i64, _c_void_p, _i64, _i64, _i64, _i64, _i64, _int,
                     _c_void_p], _int),
    "fsd_lora_linear": ([_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                         _c_void_p, _i64, _f32, _c_void_p, _i64, _i64, _i64, _i64, _i64, _int,
                         _c_void_p, ctypes.c_size_t, _c_void_p], _int),
    "fsd_lora_linear_plan": ([_i64, _i64, ctypes.c_size_t, ctypes.POINTER(_i64),
                              ctypes.POINTER(_int)], _i64),
    "fsd_lora_linear_launch": ([_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                _c_void_p, _i64, _f32, _c_void_p, _i64, _i64, _i64, _i64, _i64,
                                _int, _c_void_p, ctypes.c_size_t, _i64, _c_void_p], _int),
    "fsd_lora_linear_noalloc": ([_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                 _c_void_p, _i64, _f32, _c_void_p, _i64, _i64, _i64, _i64, _i64,
                                 _int, _c_void_p], _int),
    "fsd_graph_begin": ([_c_void_p], _int),
    "fsd_graph_end": ([_c_void_p, ctypes.POINTER(_c_void_p)], _int),
    "fsd_graph_launch": ([_c_void_p, _c_void_p], _int),
    "fsd_graph_destroy": ([_c_void_p], _int),
    "fsd_renoise": ([_c_void_p, _c_void_p, _f32, _c_void_p, _i64, _c_void_p], _int),
    "fsd_euler_step": ([_c_void_p, _c_void_p, _f32, _f32, _i64, _c_void_p], _int),
    "fsd_token_embed": ([_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i64, _c_void_p],
                        _int),
    "fsd_token_head": ([_c_void_p, _i64, _c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p],
                       _int),
    "fsd_token_head_euler": ([_c_void_p, _i64, _c_void_p, _c_void_p, _i64, _i64, _i64, _f32,
                              _f32, _c_void_p], _int),
    "fsd_mx_scale_bytes": ([_i64, _i64], ctypes.c_size_t),
    "fsd_mx_quantize": ([_c_void_p, _i64, _i64, _i64, _c_void_p, _i64, _c_void_p, _c_void_p],
                        _int),
    "fsd_mx_lora_down": ([_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _f32, _c_void_p,
                          _i64, _i64, _i64, _i64, _c_void_p], _int),
    "fsd_mx_lora_up": ([_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64,
                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p,
                        _i64, _i64, _i64, _i64, _i64, _int, _c_void_p], _int),
    "fsd_mx_lora_down_mx": ([_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _f32, _c_void_p,
                             _i64, _c_void_p, _i64, _i64, _i64, _c_void_p], _int),
    "fsd_mx_lora_up_q": ([_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64,
                          _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p,
                          _i64, _i64, _i64, _i64, _i64, _i64, _i64, _c_void_p, _i64, _c_void_p,
                          _c_void_p], _int),
    "fsd_token_embed_mx": ([_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i64, _c_void_p,
                            _i64, _c_void_p, _c_void_p], _int),
    "fsd_mx_lora_linear_workspace_bytes": ([_i64, _i64], ctypes.c_size_t),
    "fsd_mx_lora_linear_plan": ([_i64, _i64, ctypes.c_size_t, ctypes.POINTER(_i64),
                                 ctypes.POINTER(_i64)], _int),
    "fsd_mx_lora_linear": ([_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _f32, _c_void_p,
                            _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64,
                            _c_void_p, _i64, _i64, _i64, _i64, _i64, _int, _i64, _i64,
                            _c_void_p, _i64, _c_void_p, _c_void_p, ctypes.c_size_t, _c_void_p],
                           _int),
    "fsd_mx_lora_linear_launch": ([_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _f32,
                                   _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p, _i64, _c_void_p, _i64, _i64, _i64, _i64, _i64,
                                   _int, _i64, _i64, _c_void_p, _i64, _c_void_p, _c_void_p,
                                   ctypes.c_size_t, _i64, _c_void_p], _int),
    "fsd_attention_workspace_bytes": ([_i64, _i64, _i64], ctypes.c_size_t),
    "fsd_attention": ([_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p, _i64, _i64, _i64, _i64,
                       _f32, _c_void_p, ctypes.c_size_t, _c_void_p], _int),
    "fsd_mx_lora_up_swiglu_mx": ([_c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                  _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                  _i64, _c_void_p, _i64, _i64, _i64, _i64, _c_void_p], _int),
}


def lib() -> ctypes.CDLL:
    """Load libfsd.so (once).  Raises FsdError-like RuntimeError when absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"HIP library not built: {_LIB_PATH} is missing "
                               "(run __graft_entry__.build())")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().fsd_abi_version()


# ------------------------------------------------------------------ helpers
def _check(fn: str, status: int):
    if status != 0:
        raise FsdError(fn, status)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, dims=2):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dims:
        raise ValueError(f"{name} must be {dims}-D")
    if dims == 2 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    if dims == 1 and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t: torch.Tensor, name: str, shape, contiguous=False, device=None):
    """Raise ValueError unless t has exactly `shape` (and, if asked, is contiguous
    and on `device`).  The C library sees only pointers and sizes, so a wrongly
    sized buffer would be read or written out of bounds on the device: every
    tensor's extent is checked here, before any launch."""
    if tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.size(0) > 1 else max(t.stride(0), t.size(1))


# ------------------------------------------------------------------ a0 merge
def lora_merge(A_list, B_list, scales=None, out_A=None, out_B=None):
    """Rank-axis merge of fp32 adapters into bf16 A [R, K] and B [N, R]."""
    n = len(A_list)
    if n == 0 or len(B_list) != n:
        raise ValueError("need matching, non-empty adapter lists")
    K = A_list[0].shape[1]
    N = B_list[0].shape[0]
    ranks = [a.shape[0] for a in A_list]
    for a, b, r in zip(A_list, B_list, ranks):
        _need(a, "A_i", torch.float32)
        _need(b, "B_i", torch.float32)
        if not (a.is_contiguous() and b.is_contiguous()):
            raise ValueError("adapter factors must be contiguous")
        if a.shape[1] != K or b.shape != (N, r):
            raise ValueError("inconsistent adapter shapes")
    R = sum(ranks)
    dev = A_list[0].device
    for t in (*A_list, *B_list):
        if t.device != dev:
            raise ValueError("adapter factors must share one device")
    if out_A is None:
        out_A = torch.empty((R, K), dtype=torch.bfloat16, device=dev)
    if out_B is None:
        out_B = torch.empty((N, R), dtype=torch.bfloat16, device=dev)
    _need(out_A, "out_A", torch.bfloat16)
    _need(out_B, "out_B", torch.bfloat16)
    _shape(out_A, "out_A", (R, K), contiguous=True, device=dev)
    _shape(out_B, "out_B", (N, R), contiguous=True, device=dev)
    ap = (_c_void_p * n)(*[a.data_ptr() for a in A_list])
    bp = (_c_void_p * n)(*[b.data_ptr() for b in B_list])
    rk = (_i64 * n)(*ranks)
    sc = None
    if scales is not None:
        sc_arr = (ctypes.c_float * n)(*[float(s) for s in scales])
        sc = ctypes.cast(sc_arr, _c_void_p)
    st = lib().fsd_lora_merge(n, ap, bp, rk, sc, K, N, _ptr(out_A), _ptr(out_B),
                              _stream(out_A))
    _check("fsd_lora_merge", st)
    return out_A, out_B


# ------------------------------------------------------------ LoRA linear
def workspace_bytes(M: int, r: int) -> int:
    return int(lib().fsd_lora_linear_workspace_bytes(M, r))


def lora_down(X, A, scale=1.0, T=None):
    """Phase A: T = bf16(scale · X·Aᵀ)."""
    _need(X, "X", torch.bfloat16)
    _need(A, "A", torch.bfloat16)
    M, K = X.shape
    r = A.shape[0]
    _shape(A, "A", (r, K), contiguous=True, device=X.device)
    if T is None:
        T = torch.empty((M, r), dtype=torch.bfloat16, device=X.device)
    _need(T, "T", torch.bfloat16)
    _shape(T, "T", (M, r), device=X.device)
    st = lib().fsd_lora_down(_ptr(X), _ld(X), _ptr(A), float(scale), _ptr(T), _ld(T), M, K, r,
                             _stream(X))
    _check("fsd_lora_down", st)
    return T


def _out_cols(N, epilogue):
    return N // 2 if epilogue == EPI_SWIGLU else N


def _epi(epilogue):
    if isinstance(epilogue, str):
        return {"none": EPI_NONE, "swiglu": EPI_SWIGLU}[epilogue]
    return int(epilogue)


def _linear_operands(X, W0, A, B, bias, residual, epilogue, r):
    """Shape checks shared by the bf16 linear entry points (X, W0 already typed)."""
    M, K = X.shape
    N = W0.shape[0]
    dev = X.device
    _shape(W0, "W0", (N, K), contiguous=True, device=dev)
    if r:
        if A is not None:
            _need(A, "A", torch.bfloat16)
            _shape(A, "A", (r, K), contiguous=True, device=dev)
        _need(B, "B", torch.bfloat16)
        _shape(B, "B", (N, r), contiguous=True, device=dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, dims=1)
        _shape(bias, "bias", (N,), device=dev)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16)
        _shape(residual, "residual", (M, _out_cols(N, epilogue)), device=dev)


def lora_up(X, W0, T, B, bias=None, residual=None, epilogue=EPI_NONE, out=None):
    """Phase B: Y = epi([X | T]·[W0 | B]ᵀ + bias) (+ residual)."""
    epilogue = _epi(epilogue)
    _need(X, "X", torch.bfloat16)
    _need(W0, "W0", torch.bfloat16)
    M, K = X.shape
    N = W0.shape[0]
    r = 0 if B is None else B.shape[1]
    _linear_operands(X, W0, None, B, bias, residual, epilogue, r)
    if r:
        _need(T, "T", torch.bfloat16)
        _shape(T, "T", (M, r), device=X.device)
    if out is None:
        out = torch.empty((M, _out_cols(N, epilogue)), dtype=torch.bfloat16, device=X.device)
    _need(out, "out", torch.bfloat16)
    _shape(out, "out", (M, _out_cols(N, epilogue)), device=X.device)
    st = lib().fsd_lora_up(_ptr(X), _ld(X), _ptr(W0), _ptr(T) if r else None,
                           _ld(T) if r else 0, _ptr(B) if r else None, _ptr(bias),
                           _ptr(residual), _ld(residual) if residual is not None else 0,
                           _ptr(out), _ld(out), M, N, K, r, epilogue, _stream(X))
    _check("fsd_lora_up", st)
    return out


def lora_linear_plan(M: int, r: int, ws_bytes: int):
    """(launches, rows per chunk, schedule) of fsd_lora_linear (see include/fsd.h)."""
    R = _i64(0)
    sched = _int(0)
    n = lib().fsd_lora_linear_plan(int(M), int(r), int(ws_bytes), ctypes.byref(R),
                                   ctypes.byref(sched))
    if n < 0:
        raise ValueError("negative M or r")
    return int(n), int(R.value), int(sched.value)


def lora_linear(X, W0, A, B, scale=1.0, bias=None, residual=None, epilogue=EPI_NONE,
                out=None, workspace=None, on_launch=None):
    """Y = epi(X·W0ᵀ + scale·(X·Aᵀ)·Bᵀ + bias) (+ residual): phase A then phase B,
    chunked through a small workspace of T (fsd_lora_linear).

    workspace: uint8 device tensor; default: workspace_bytes(M, r) (the library's
    preferred size, 50.1 MB at r = 576 for M > 43,520).
    on_launch: optional callable(index) run on the host before each kernel launch
    of the schedule (e.g. to record timing events between launches); the
    launches are then issued one by one through fsd_lora_linear_launch."""
    epilogue = _epi(epilogue)
    _need(X, "X", torch.bfloat16)
    _need(W0, "W0", torch.bfloat16)
    M, K = X.shape
    N = W0.shape[0]
    r = 0 if A is None else A.shape[0]
    _linear_operands(X, W0, A, B, bias, residual, epilogue, r)
    if out is None:
        out = torch.empty((M, _out_cols(N, epilogue)), dtype=torch.bfloat16, device=X.device)
    _need(out, "out", torch.bfloat16)
    _shape(out, "out", (M, _out_cols(N, epilogue)), device=X.device)
    if workspace is not None and (workspace.device != X.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on X's device")
    if workspace is None and r:
        workspace = torch.empty(max(workspace_bytes(M, r), 16), dtype=torch.uint8,
                                device=X.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(X), _ld(X), _ptr(W0), _ptr(A) if r else None, _ptr(B) if r else None,
            _ptr(bias), _ptr(residual), _ld(residual) if residual is not None else 0,
            float(scale), _ptr(out), _ld(out), M, N, K, r, epilogue, _ptr(workspace), ws_bytes)
    if on_launch is None:
        st = lib().fsd_lora_linear(*args, _stream(X))
        _check("fsd_lora_linear", st)
        return out
    n, _, _ = lora_linear_plan(M, r, ws_bytes)
    for i in range(n):
        on_launch(i)
        st = lib().fsd_lora_linear_launch(*args, i, _stream(X))
        _check("fsd_lora_linear_launch", st)
    return out


def lora_linear_noalloc(X, W0, A, B, scale=1.0, bias=None, residual=None, epilogue=EPI_NONE,
                        out=None):
    """lora_linear with T in the library's per-GPU scratch (fsd_lora_linear_noalloc):
    no device memory is allocated for the call (pass `out` to allocate nothing at
    all).  Calls that overlap on one GPU share the scratch and must be ordered."""
    epilogue = _epi(epilogue)
    _need(X, "X", torch.bfloat16)
    _need(W0, "W0", torch.bfloat16)
    M, K = X.shape
    N = W0.shape[0]
    r = 0 if A is None else A.shape[0]
    _linear_operands(X, W0, A, B, bias, residual, epilogue, r)
    if out is None:
        out = torch.empty((M, _out_cols(N, epilogue)), dtype=torch.bfloat16, device=X.device)
    _need(out, "out", torch.bfloat16)
    _shape(out, "out", (M, _out_cols(N, epilogue)), device=X.device)
    st = lib().fsd_lora_linear_noalloc(
        _ptr(X), _ld(X), _ptr(W0), _ptr(A) if r else None, _ptr(B) if r else None, _ptr(bias),
        _ptr(residual), _ld(residual) if residual is not None else 0, float(scale), _ptr(out),
        _ld(out), M, N, K, r, epilogue, _stream(X))
    _check("fsd_lora_linear_noalloc", st)
    return out


# ------------------------------------------------------------ sampler
def renoise(u, eps, sigma, out=None):
    """z = (1 - sigma)·u + sigma·eps (fp32, any shape, contiguous)."""
    for t, nm in ((u, "u"), (eps, "eps")):
        if t.device.type != "cuda" or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous fp32 GPU tensor")
    if u.shape != eps.shape or u.device != eps.device:
        raise ValueError("u and eps shapes or devices differ")
    if out is None:
        out = torch.empty_like(u)
    if (out.shape != u.shape or out.dtype != torch.float32 or not out.is_contiguous()
            or out.device != u.device):
        raise ValueError("out must be a contiguous fp32 tensor shaped like u")
    st = lib().fsd_renoise(_ptr(u), _ptr(eps), float(sigma), _ptr(out), u.numel(), _stream(u))
    _check("fsd_renoise", st)
    return out


def euler_step(z, v, sigma, sigma_next):
    """z <- z + (sigma_next - sigma)·v, in place."""
    for t, nm in ((z, "z"), (v, "v")):
        if t.device.type != "cuda" or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous fp32 GPU tensor")
    if z.numel() != v.numel() or z.device != v.device:
        raise ValueError("z and v sizes or devices differ")
    st = lib().fsd_euler_step(_ptr(z), _ptr(v), float(sigma), float(sigma_next), z.numel(),
                              _stream(z))
    _check("fsd_euler_step", st)
    return z


# ------------------------------------------------------------ stand-in
def token_embed(z, E, out=None):
    """X = bf16(z·Eᵀ): z fp32 [M, C], E bf16 [D, C] -> X bf16 [M, D]."""
    if z.device.type != "cuda" or z.dtype != torch.float32 or not z.is_contiguous() or z.dim() != 2:
        raise ValueError("z must be a contiguous fp32 [M, C] GPU tensor")
    _need(E, "E", torch.bfloat16)
    M, C = z.shape
    D = E.shape[0]
    _shape(E, "E", (D, C), contiguous=True, device=z.device)
    if out is None:
        out = torch.empty((M, D), dtype=torch.bfloat16, device=z.device)
    _need(out, "out", torch.bfloat16)
    _shape(out, "out", (M, D), device=z.device)
    st = lib().fsd_token_embed(_ptr(z), _ptr(E), _ptr(out), _ld(out), M, C, D, _stream(z))
    _check("fsd_token_embed", st)
    return out


def token_embed_mx(z, E, out=None, Xq=None, Xs=None):
    """token_embed that also writes X's MXFP8 form: returns (X bf16 [M, D], Xq uint8
    [M, D], Xs scales), Xq/Xs the bytes mx_quantize(X) would make.  D % 128 == 0."""
    if z.device.type != "cuda" or z.dtype != torch.float32 or not z.is_contiguous() or z.dim() != 2:
        raise ValueError("z must be a contiguous fp32 [M, C] GPU tensor")
    _need(E, "E", torch.bfloat16)
    M, C = z.shape
    D = E.shape[0]
    _shape(E, "E", (D, C), contiguous=True, device=z.device)
    if out is None:
        out = torch.empty((M, D), dtype=torch.bfloat16, device=z.device)
    if Xq is None:
        Xq = torch.empty((M, mx_padded_k(D)), dtype=torch.uint8, device=z.device)
    if Xs is None:
        Xs = torch.empty(max(mx_scale_bytes(M, D), 4), dtype=torch.uint8, device=z.device)
    _need(out, "out", torch.bfloat16)
    _shape(out, "out", (M, D), device=z.device)
    _need(Xq, "Xq", torch.uint8)
    _shape(Xq, "Xq", (M, mx_padded_k(D)), device=z.device)
    _need_scales(Xs, "Xs", M, mx_padded_k(D))
    if Xs.device != z.device:
        raise ValueError("Xs must be on z's device")
    st = lib().fsd_token_embed_mx(_ptr(z), _ptr(E), _ptr(out), _ld(out), M, C, D, _ptr(Xq),
                                  _ld(Xq), _ptr(Xs), _stream(z))
    _check("fsd_token_embed_mx", st)
    return out, Xq, Xs


def token_head(H, P, out=None):
    """v = H·Pᵀ: H bf16 [M, D], P bf16 [C, D] -> v fp32 [M, C]."""
    _need(H, "H", torch.bfloat16)
    _need(P, "P", torch.bfloat16)
    M, D = H.shape
    C = P.shape[0]
    _shape(P, "P", (C, D), contiguous=True, device=H.device)
    if out is None:
        out = torch.empty((M, C), dtype=torch.float32, device=H.device)
    if out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor")
    _shape(out, "out", (M, C), device=H.device)
    st = lib().fsd_token_head(_ptr(H), _ld(H), _ptr(P), _ptr(out), M, D, C, _stream(H))
    _check("fsd_token_head", st)
    return out


def token_head_euler(H, P, z, sigma, sigma_next):
    """z += (sigma_next - sigma)·(H·Pᵀ) in place: H bf16 [M, D], P bf16 [C, D], z fp32 [M, C]."""
    _need(H, "H", torch.bfloat16)
    _need(P, "P", torch.bfloat16)
    M, D = H.shape
    C = P.shape[0]
    _shape(P, "P", (C, D), contiguous=True, device=H.device)
    if z.dtype != torch.float32 or not z.is_contiguous():
        raise ValueError("z must be a contiguous fp32 [M, C] tensor")
    _shape(z, "z", (M, C), device=H.device)
    st = lib().fsd_token_head_euler(_ptr(H), _ld(H), _ptr(P), _ptr(z), M, D, C, float(sigma),
                                    float(sigma_next), _stream(H))
    _check("fsd_token_head_euler", st)
    return z


def mx_padded_k(K: int) -> int:
    """Row length of MXFP8 elements: K rounded up to one GEMM K step (128)."""
    return (K + 127) // 128 * 128


def mx_quantize(X, Q=None, S=None):
    """MXFP8 of X bf16 [M, K] (K % 32 == 0): returns (Q uint8 [M, Kp], S uint8 scales)."""
    _need(X, "X", torch.bfloat16)
    M, K = X.shape
    Kp = mx_padded_k(K)
    if Q is None:
        Q = torch.empty((M, Kp), dtype=torch.uint8, device=X.device)
    if S is None:
        S = torch.empty(int(lib().fsd_mx_scale_bytes(M, K)), dtype=torch.uint8, device=X.device)
    _need(Q, "Q", torch.uint8)
    _shape(Q, "Q", (M, Kp), device=X.device)
    _need_scales(S, "S", M, Kp)
    if S.device != X.device:
        raise ValueError("S must be on X's device")
    st = lib().fsd_mx_quantize(_ptr(X), _ld(X), M, K, _ptr(Q), Q.stride(0), _ptr(S), _stream(X))
    _check("fsd_mx_quantize", st)
    return Q, S


def mx_scale_bytes(M: int, K: int) -> int:
    """Bytes of the scale array of M rows of K elements."""
    return int(lib().fsd_mx_scale_bytes(M, K))


def mx_scale_offsets(M: int, K: int) -> np.ndarray:
    """Byte offset in the scale array of the scale of (row m, 32-element block b).

    int64 [M, Kp/32].  Scales are grouped by 128-element step t and 64-row group
    g; within a group, byte i of 32-bit word 16·b + r is row 64g + 16i + r.
    """
    Kp = mx_padded_k(K)
    Mp = (M + 255) // 256 * 256
    m = np.arange(M, dtype=np.int64)[:, None]
    b = np.arange(Kp // 32, dtype=np.int64)[None, :]
    return (((b >> 2) * (Mp >> 6) + (m >> 6)) * 64 + (b & 3) * 16 + (m & 15)) * 4 + ((m >> 4) & 3)


def mx_pack_scales(s_rows, K: int) -> torch.Tensor:
    """Host uint8 scales [M, Kp/32] (row-major, one byte per block) -> the scale
    array layout (CPU uint8 tensor; padding rows hold 127)."""
    s_rows = np.asarray(s_rows, dtype=np.uint8)
    M = s_rows.shape[0]
    out = np.full(max(mx_scale_bytes(M, K), 0), 127, np.uint8)
    out[mx_scale_offsets(M, K)] = s_rows
    return torch.from_numpy(out)


def mx_unpack_scales(S, M: int, K: int) -> np.ndarray:
    """Scale array (any device) -> host uint8 [M, Kp/32], one byte per (row, block)."""
    flat = S.detach().cpu().numpy() if isinstance(S, torch.Tensor) else np.asarray(S)
    return flat[mx_scale_offsets(M, K)]


def _need_scales(S, name, rows, Kp):
    if not isinstance(S, torch.Tensor) or S.device.type != "cuda" or S.dtype != torch.uint8:
        raise TypeError(f"{name} must be a uint8 GPU tensor")
    if not S.is_contiguous() or S.numel() < mx_scale_bytes(rows, Kp):
        raise ValueError(f"{name} must hold the scales of {rows} rows of {Kp} elements")


def mx_lora_down(Xq, Xs, Aq, As, scale=1.0, T=None):
    """Phase A on MXFP8 operands: T = bf16(scale · deq(Xq)·deq(Aq)ᵀ).

    Xq uint8 [M, Kp] with scales Xs; Aq uint8 [r, Kp] (contiguous) with scales As.
    """
    _need(Xq, "Xq", torch.uint8)
    _need(Aq, "Aq", torch.uint8)
    M, Kp = Xq.shape
    r = Aq.shape[0]
    if Aq.shape[1] != Kp or not Aq.is_contiguous():
        raise ValueError("Aq must be a contiguous [r, Kp] tensor with Xq's Kp")
    _need_scales(Xs, "Xs", M, Kp)
    _need_scales(As, "As", r, Kp)
    for t, nm in ((Aq, "Aq"), (Xs, "Xs"), (As, "As")):
        if t.device != Xq.device:
            raise ValueError(f"{nm} must be on Xq's device")
    if T is None:
        T = torch.empty((M, r), dtype=torch.bfloat16, device=Xq.device)
    _need(T, "T", torch.bfloat16)
    _shape(T, "T", (M, r), device=Xq.device)
    st = lib().fsd_mx_lora_down(_ptr(Xq), _ld(Xq), _ptr(Xs), _ptr(Aq), _ptr(As), float(scale),
                                _ptr(T), _ld(T), M, Kp, r, _stream(Xq))
    _check("fsd_mx_lora_down", st)
    return T


def _mx_up_operands(Xq, Xs, W0q, W0s, Tq, Ts, Bq, Bs, bias):
    _need(Xq, "Xq", torch.uint8)
    _need(W0q, "W0q", torch.uint8)
    M, Kp = Xq.shape
    N = W0q.shape[0]
    if W0q.shape[1] != Kp or not W0q.is_contiguous():
        raise ValueError("W0q must be a contiguous [N, Kp] tensor with Xq's Kp")
    _need_scales(Xs, "Xs", M, Kp)
    _need_scales(W0s, "W0s", N, Kp)
    rp = 0 if Bq is None else Bq.shape[1]
    if rp:
        _need(Tq, "Tq", torch.uint8)
        _need(Bq, "Bq", torch.uint8)
        if Tq.shape != (M, rp) or Bq.shape[0] != N or not Bq.is_contiguous():
            raise ValueError("Tq must be [M, rp] and Bq a contiguous [N, rp]")
        _need_scales(Ts, "Ts", M, rp)
        _need_scales(Bs, "Bs", N, rp)
    if bias is not None:
        _need(bias, "bias", torch.float32, dims=1)
        _shape(bias, "bias", (N,), device=Xq.device)
    for t, nm in ((W0q, "W0q"), (Xs, "Xs"), (W0s, "W0s"), (Tq, "Tq"), (Ts, "Ts"), (Bq, "Bq"),
                  (Bs, "Bs")):
        if t is not None and t.device != Xq.device:
            raise ValueError(f"{nm} must be on Xq's device")
    ops = (_ptr(Xq), _ld(Xq), _ptr(Xs), _ptr(W0q), _ptr(W0s), _ptr(Tq) if rp else None,
           _ld(Tq) if rp else 0, _ptr(Ts) if rp else None, _ptr(Bq) if rp else None,
           _ptr(Bs) if rp else None, _ptr(bias))
    return M, N, Kp, rp, ops


def mx_lora_up(Xq, Xs, W0q, W0s, Tq=None, Ts=None, Bq=None, Bs=None, bias=None,
               residual=None, epilogue=EPI_NONE, out=None):
    """Phase B on MXFP8 operands: Y = epi([Xq | Tq]·[W0q | Bq]ᵀ (dequantized) + bias) (+ residual).

    Xq uint8 [M, Kp]; W0q uint8 [N, Kp] (contiguous); Tq uint8 [M, rp] and Bq uint8
    [N, rp] (contiguous), rp a multiple of 128, or None for no LoRA term; Xs, W0s,
    Ts, Bs their scale arrays.
    """
    epilogue = _epi(epilogue)
    M, N, Kp, rp, ops = _mx_up_operands(Xq, Xs, W0q, W0s, Tq, Ts, Bq, Bs, bias)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16)
        _shape(residual, "residual", (M, _out_cols(N, epilogue)), device=Xq.device)
    if out is None:
        out = torch.empty((M, _out_cols(N, epilogue)), dtype=torch.bfloat16, device=Xq.device)
    _need(out, "out", torch.bfloat16)
    _shape(out, "out", (M, _out_cols(N, epilogue)), device=Xq.device)
    st = lib().fsd_mx_lora_up(*ops, _ptr(residual),
                              _ld(residual) if residual is not None else 0, _ptr(out), _ld(out),
                              M, N, Kp, rp, epilogue, _stream(Xq))
    _check("fsd_mx_lora_up", st)
    return out


def mx_lora_up_swiglu_mx(Xq, Xs, W0q, W0s, Tq=None, Ts=None, Bq=None, Bs=None, bias=None,
                         Hq=None, Hs=None):
    """Phase B with SwiGLU, its output H quantized to MXFP8 in the same pass.

    Returns (Hq uint8 [M, N/2], Hs scales), the bytes mx_quantize would make of the
    bf16 output of mx_lora_up(..., epilogue="swiglu").  N % 256 == 0.
    """
    M, N, Kp, rp, ops = _mx_up_operands(Xq, Xs, W0q, W0s, Tq, Ts, Bq, Bs, bias)
    F = N // 2
    if Hq is None:
        Hq = torch.empty((M, F), dtype=torch.uint8, device=Xq.device)
    if Hs is None:
        Hs = torch.empty(max(mx_scale_bytes(M, F), 4), dtype=torch.uint8, device=Xq.device)
    _need(Hq, "Hq", torch.uint8)
    _shape(Hq, "Hq", (M, F), device=Xq.device)
    _need_scales(Hs, "Hs", M, F)
    st = lib().fsd_mx_lora_up_swiglu_mx(*ops, _ptr(Hq), _ld(Hq), _ptr(Hs), M, N, Kp, rp,
                                        _stream(Xq))
    _check("fsd_mx_lora_up_swiglu_mx", st)
    return Hq, Hs


def mx_lora_down_mx(Xq, Xs, Aq, As, scale=1.0, Tq=None, Ts=None):
    """Phase A on MXFP8 operands whose T leaves only as MXFP8: returns (Tq uint8
    [M, rp], Ts scales), the bytes mx_quantize(mx_lora_down(...)) would make.
    r = Aq.shape[0] must be a multiple of 32; rp = r rounded up to 128."""
    _need(Xq, "Xq", torch.uint8)
    _need(Aq, "Aq", torch.uint8)
    M, Kp = Xq.shape
    r = Aq.shape[0]
    if Aq.shape[1] != Kp or not Aq.is_contiguous():
        raise ValueError("Aq must be a contiguous [r, Kp] tensor with Xq's Kp")
    _need_scales(Xs, "Xs", M, Kp)
    _need_scales(As, "As", r, Kp)
    rp = mx_padded_k(r)
    if Tq is None:
        Tq = torch.empty((M, rp), dtype=torch.uint8, device=Xq.device)
    if Ts is None:
        Ts = torch.empty(max(mx_scale_bytes(M, r), 4), dtype=torch.uint8, device=Xq.device)
    _need(Tq, "Tq", torch.uint8)
    _shape(Tq, "Tq", (M, rp), device=Xq.device)
    _need_scales(Ts, "Ts", M, rp)
    for t, nm in ((Aq, "Aq"), (Xs, "Xs"), (As, "As"), (Ts, "Ts")):
        if t.device != Xq.device:
            raise ValueError(f"{nm} must be on Xq's device")
    st = lib().fsd_mx_lora_down_mx(_ptr(Xq), _ld(Xq), _ptr(Xs), _ptr(Aq), _ptr(As), float(scale),
                                   _ptr(Tq), _ld(Tq), _ptr(Ts), M, Kp, r, _stream(Xq))
    _check("fsd_mx_lora_down_mx", st)
    return Tq, Ts


def mx_lora_up_q(Xq, Xs, W0q, W0s, Tq=None, Ts=None, Bq=None, Bs=None, bias=None,
                 residual=None, out=None, cols=None, Yq=None, Ys=None):
    """mx_lora_up (plain epilogue) that also writes the MXFP8 form of the output's
    columns cols = (q0, q1) (default: all): returns (Y, Yq uint8 [M, q1 - q0 rounded
    up to 128], Ys), Yq/Ys the bytes mx_quantize(Y[:, q0:q1]) would make."""
    M, N, Kp, rp, ops = _mx_up_operands(Xq, Xs, W0q, W0s, Tq, Ts, Bq, Bs, bias)
    q0, q1 = (0, N) if cols is None else (int(cols[0]), int(cols[1]))
    qkp = mx_padded_k(q1 - q0)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16)
        _shape(residual, "residual", (M, N), device=Xq.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=Xq.device)
    if Yq is None:
        Yq = torch.empty((M, qkp), dtype=torch.uint8, device=Xq.device)
    if Ys is None:
        Ys = torch.empty(max(mx_scale_bytes(M, q1 - q0), 4), dtype=torch.uint8, device=Xq.device)
    _need(out, "out", torch.bfloat16)
    _shape(out, "out", (M, N), device=Xq.device)
    _need(Yq, "Yq", torch.uint8)
    _shape(Yq, "Yq", (M, qkp), device=Xq.device)
    _need_scales(Ys, "Ys", M, qkp)
    if Ys.device != Xq.device:
        raise ValueError("Ys must be on Xq's device")
    st = lib().fsd_mx_lora_up_q(*ops, _ptr(residual),
                                _ld(residual) if residual is not None else 0, _ptr(out), _ld(out),
                                M, N, Kp, rp, q0, q1, _ptr(Yq), _ld(Yq), _ptr(Ys), _stream(Xq))
    _check("fsd_mx_lora_up_q", st)
    return out, Yq, Ys


def mx_workspace_bytes(M: int, r: int) -> int:
    """Preferred workspace of mx_lora_linear: two chunks of MXFP8 T."""
    return int(lib().fsd_mx_lora_linear_workspace_bytes(M, r))


def mx_lora_linear_plan(M: int, r: int, ws_bytes: int):
    """(launches, chunk rows) of mx_lora_linear for M rows at rank r."""
    n, R = _i64(0), _i64(0)
    st = lib().fsd_mx_lora_linear_plan(M, r, ws_bytes, ctypes.byref(n), ctypes.byref(R))
    _check("fsd_mx_lora_linear_plan", st)
    return n.value, R.value


def mx_lora_linear(Xq, Xs, Aq, As, W0q, W0s, Bq, Bs, scale=1.0, bias=None, residual=None,
                   out=None, epilogue=EPI_NONE, cols=None, Yq=None, Ys=None, workspace=None,
                   on_launch=None):
    """The whole MXFP8 LoRA linear in row chunks (fsd_mx_lora_linear): T = the MXFP8
    of bf16(scale·X·Aᵀ) per chunk in the workspace, then phase B.

    epilogue "none": returns out (bf16 [M, N]); with Yq/Ys (or cols) also the MXFP8
    of out[:, q0:q1], returned as (out, Yq, Ys).  epilogue "swiglu": out bf16 [M, N/2],
    or, with Yq/Ys and out=None, the MXFP8 of H only, returned as (Yq, Ys).
    on_launch: optional callable(index) run before each launch (launches then go one
    by one through fsd_mx_lora_linear_launch)."""
    epilogue = _epi(epilogue)
    for t, nm in ((Xq, "Xq"), (Aq, "Aq"), (W0q, "W0q"), (Bq, "Bq")):
        _need(t, nm, torch.uint8)
    M, Kp = Xq.shape
    r, N, rp = Aq.shape[0], W0q.shape[0], mx_padded_k(Aq.shape[0])
    _shape(Aq, "Aq", (r, Kp), contiguous=True, device=Xq.device)
    _shape(W0q, "W0q", (N, Kp), contiguous=True, device=Xq.device)
    _shape(Bq, "Bq", (N, rp), contiguous=True, device=Xq.device)
    for S_, nm, rows, k in ((Xs, "Xs", M, Kp), (As, "As", r, Kp), (W0s, "W0s", N, Kp),
                            (Bs, "Bs", N, rp)):
        _need_scales(S_, nm, rows, k)
        if S_.device != Xq.device:
            raise ValueError(f"{nm} must be on Xq's device")
    if bias is not None:
        _need(bias, "bias", torch.float32, dims=1)
        _shape(bias, "bias", (N,), device=Xq.device)
    swiglu = epilogue == EPI_SWIGLU
    nout = N // 2 if swiglu else N
    quant = Yq is not None or Ys is not None or cols is not None
    q0, q1 = (0, nout) if cols is None else (int(cols[0]), int(cols[1]))
    if quant:
        qkp = mx_padded_k(q1 - q0)
        if Yq is None:
            Yq = torch.empty((M, qkp), dtype=torch.uint8, device=Xq.device)
        if Ys is None:
            Ys = torch.empty(max(mx_scale_bytes(M, q1 - q0), 4), dtype=torch.uint8,
                             device=Xq.device)
        _need(Yq, "Yq", torch.uint8)
        _shape(Yq, "Yq", (M, qkp), device=Xq.device)
        _need_scales(Ys, "Ys", M, qkp)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16)
        _shape(residual, "residual", (M, nout), device=Xq.device)
    if out is None and not (swiglu and quant):
        out = torch.empty((M, nout), dtype=torch.bfloat16, device=Xq.device)
    if out is not None:
        _need(out, "out", torch.bfloat16)
        _shape(out, "out", (M, nout), device=Xq.device)
    if workspace is None:
        workspace = torch.empty(max(mx_workspace_bytes(M, r), 16), dtype=torch.uint8,
                                device=Xq.device)
    if workspace.device != Xq.device or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on Xq's device")
    args = [_ptr(Xq), _ld(Xq), _ptr(Xs), _ptr(Aq), _ptr(As), float(scale), _ptr(W0q), _ptr(W0s),
            _ptr(Bq), _ptr(Bs), _ptr(bias),
            _ptr(residual), _ld(residual) if residual is not None else 0,
            _ptr(out) if out is not None else None, _ld(out) if out is not None else 0,
            M, N, Kp, r, epilogue, q0 if quant else 0, q1 if quant else 0,
            _ptr(Yq) if quant else None, _ld(Yq) if quant else 0, _ptr(Ys) if quant else None,
            _ptr(workspace), workspace.numel()]
    if on_launch is None:
        st = lib().fsd_mx_lora_linear(*args, _stream(Xq))
        _check("fsd_mx_lora_linear", st)
    else:
        n, _ = mx_lora_linear_plan(M, r, workspace.numel()) if M else (0, 0)
        for i in range(n):
            on_launch(i)
            st = lib().fsd_mx_lora_linear_launch(*args, i, _stream(Xq))
            _check("fsd_mx_lora_linear_launch", st)
    if swiglu and quant and out is None:
        return Yq, Ys
    if quant:
        return out, Yq, Ys
    return out


# ------------------------------------------------------------ attention
def attention_workspace_bytes(S: int, H: int, D: int = 128) -> int:
    return int(lib().fsd_attention_workspace_bytes(S, H, D))


def attention(Q, K, V, heads, scale=None, out=None, workspace=None):
    """O = softmax(Q·Kᵀ·scale)·V per head.  Q, K, V bf16 [S, heads·128] views with
    one row stride (e.g. slices of a QKV output); returns O bf16 [S, heads·128]."""
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, nm, torch.bfloat16)
    S, HD = Q.shape
    if K.shape != (S, HD) or V.shape != (S, HD):
        raise ValueError("Q, K and V must have one shape")
    if not (_ld(Q) == _ld(K) == _ld(V)):
        raise ValueError("Q, K and V must share one row stride")
    if HD % heads:
        raise ValueError("columns must be heads x head_dim")
    D = HD // heads
    scale = 1.0 / D ** 0.5 if scale is None else float(scale)
    if K.device != Q.device or V.device != Q.device:
        raise ValueError("Q, K and V must share one device")
    if out is None:
        out = torch.empty((S, HD), dtype=torch.bfloat16, device=Q.device)
    _need(out, "out", torch.bfloat16)
    _shape(out, "out", (S, HD), device=Q.device)
    if workspace is not None and (workspace.device != Q.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on Q's device")
    if workspace is None:
        workspace = torch.empty(max(attention_workspace_bytes(S, heads, D), 16), dtype=torch.uint8,
                                device=Q.device)
    st = lib().fsd_attention(_ptr(Q), _ptr(K), _ptr(V), _ld(Q), _ptr(out), _ld(out), S, heads, D,
                             float(scale), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(Q))
    _check("fsd_attention", st)
    return out


# ------------------------------------------------------------ step graphs
class StepGraph:
    """A HIP graph of the launches this library enqueues on one stream between
    begin() and end() (fsd_graph_begin / fsd_graph_end), replayed by launch().

    with StepGraph.capture(stream) as g:   # stream: a torch.cuda.Stream
        ... library calls under torch.cuda.stream(stream) ...
    g.launch(stream)
    """

    def __init__(self):
        self._g = None

    @classmethod
    def capture(cls, stream):
        return _Capture(cls(), stream)

    def launch(self, stream=None):
        if self._g is None:
            raise RuntimeError("no captured graph")
        s = torch.cuda.current_stream() if stream is None else stream
        _check("fsd_graph_launch", lib().fsd_graph_launch(self._g, ctypes.c_void_p(s.cuda_stream)))

    def close(self):
        if self._g is not None:
            lib().fsd_graph_destroy(self._g)
            self._g = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class _Capture:
    def __init__(self, graph, stream):
        self.graph, self.stream = graph, stream
        self._ctx = torch.cuda.stream(stream)

    def __enter__(self):
        self._ctx.__enter__()
        _check("fsd_graph_begin", lib().fsd_graph_begin(ctypes.c_void_p(self.stream.cuda_stream)))
        return self.graph

    def __exit__(self, et, ev, tb):
        h = _c_void_p()
        st = lib().fsd_graph_end(ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(h))
        self._ctx.__exit__(et, ev, tb)
        if et is None:
            _check("fsd_graph_end", st)
            self.graph._g = h.value
        elif h.value:
            lib().fsd_graph_destroy(h)
        return False
