"""fp64 CPU oracle of the refiner's hot path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  It wraps ``oracle.c`` (plain C, built with gcc)
through ctypes and shares no code with the HIP library.

Sources:
  [EN] "Open-H3-Regenerate-2K: High-Resolution Video Refinement with Few-Step
       Diffusion" (agientry.com, English article)
  [CW] "Open-H3-Regenerate-2K：MiniMax H3 的开源 4K 精修方案" (comfyui-wiki.com)
  [IC] "Open-H3-Regenerate-2K-IC:草稿留在上下文里,2K 与 4K 重绘仍对着原来的脸、口型和字"
       (wujieai.com)

Functions take numpy arrays; bf16 tensors are passed as float32 arrays holding
the exact bf16 values.  Every result is float64.

Pins: see tests/test_oracle_*.py.  Parity of the velocity stand-in is only
partially pinned (special cases); everything else is pinned by closed forms,
exact rational arithmetic or an independent library routine.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None

F32P = ctypes.POINTER(ctypes.c_float)
F64P = ctypes.POINTER(ctypes.c_double)
I64P = ctypes.POINTER(ctypes.c_int64)
U16P = ctypes.POINTER(ctypes.c_uint16)


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (plain -O2, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", _SRC,
                               "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


class LoraLayer(ctypes.Structure):
    _fields_ = [("W0", F32P), ("A", F32P), ("B", F32P), ("bias", F32P),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("r", ctypes.c_int64),
                ("scale", ctypes.c_double)]


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.oracle_bf16_bits.restype = ctypes.c_uint16
        L.oracle_bf16_bits.argtypes = [ctypes.c_float]
        L.oracle_merge.argtypes = [ctypes.c_int, ctypes.POINTER(F32P), ctypes.POINTER(F32P),
                                   I64P, F64P, ctypes.c_int64, ctypes.c_int64, F64P, F64P]
        L.oracle_merge_bf16.argtypes = [ctypes.c_int, ctypes.POINTER(F32P), ctypes.POINTER(F32P),
                                        I64P, F32P, ctypes.c_int64, ctypes.c_int64, U16P, U16P]
        L.oracle_lora_linear_rows.argtypes = [
            F32P, ctypes.c_int64, I64P, ctypes.c_int64, F32P, F32P, F32P, F32P, F32P,
            ctypes.c_int64, ctypes.c_double, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, F64P, ctypes.c_int]
        L.oracle_lora_linear_drows.argtypes = [
            F64P, ctypes.c_int64, ctypes.c_int64, F32P, F32P, F32P, ctypes.c_double,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, F64P, ctypes.c_int]
        L.oracle_embed_rows.argtypes = [F32P, ctypes.c_int64, F32P, ctypes.c_int64,
                                        ctypes.c_int64, F64P]
        L.oracle_head_rows.argtypes = [F32P, ctypes.c_int64, ctypes.c_int64, F32P,
                                       ctypes.c_int64, ctypes.c_int64, F64P]
        L.oracle_renoise.argtypes = [F32P, F32P, ctypes.c_double, F64P, ctypes.c_int64]
        L.oracle_euler_step.argtypes = [F64P, F64P, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_int64]
        L.oracle_sampler_exact_velocity.argtypes = [F32P, F32P, F64P, ctypes.c_int, F64P,
                                                    ctypes.c_int64]
        L.oracle_standin_refine.argtypes = [
            F32P, F32P, ctypes.c_int64, F64P, ctypes.c_int, F32P, F32P, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(LoraLayer), F64P, F64P, ctypes.c_int]
        L.oracle_standin_velocity.argtypes = [
            F64P, ctypes.c_int64, F32P, F32P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.POINTER(LoraLayer), F64P]
        _lib = L
    return _lib


# ----------------------------------------------------------------- helpers
def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a, t):
    return None if a is None else a.ctypes.data_as(t)


def default_threads() -> int:
    """Host threads for the oracle: OMP_NUM_THREADS if set, else min(cores, 16)."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(os.cpu_count() or 1, 16))


def _nt(n):
    return int(n) if n and n > 0 else default_threads()


def bf16_bits(x) -> np.ndarray:
    """Round-to-nearest-even of float32 values to bfloat16, as uint16 bit patterns."""
    x = _f32(x).ravel()
    f = lib().oracle_bf16_bits
    return np.array([f(float(v)) for v in x], dtype=np.uint16)


def bf16_value(bits) -> np.ndarray:
    """Float32 value of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


# ----------------------------------------------------------------- a0 merge
def merge(A_list, B_list, scales=None):
    """fp64 rank-axis merge: A = [A_0; A_1; ...], B = [s_0 B_0 | s_1 B_1 | ...]."""
    n = len(A_list)
    A_list = [_f32(a) for a in A_list]
    B_list = [_f32(b) for b in B_list]
    ranks = np.array([a.shape[0] for a in A_list], dtype=np.int64)
    K = A_list[0].shape[1]
    N = B_list[0].shape[0]
    R = int(ranks.sum())
    A = np.empty((R, K), np.float64)
    B = np.empty((N, R), np.float64)
    ap = (F32P * n)(*[a.ctypes.data_as(F32P) for a in A_list])
    bp = (F32P * n)(*[b.ctypes.data_as(F32P) for b in B_list])
    sc = None if scales is None else _f64(scales)
    lib().oracle_merge(n, ap, bp, ranks.ctypes.data_as(I64P), _p(sc, F64P), K, N,
                       A.ctypes.data_as(F64P), B.ctypes.data_as(F64P))
    return A, B


def merge_bf16(A_list, B_list, scales=None):
    """Bit-exact bf16 storage form of the merge (uint16 bit patterns)."""
    n = len(A_list)
    A_list = [_f32(a) for a in A_list]
    B_list = [_f32(b) for b in B_list]
    ranks = np.array([a.shape[0] for a in A_list], dtype=np.int64)
    K = A_list[0].shape[1]
    N = B_list[0].shape[0]
    R = int(ranks.sum())
    A = np.empty((R, K), np.uint16)
    B = np.empty((N, R), np.uint16)
    ap = (F32P * n)(*[a.ctypes.data_as(F32P) for a in A_list])
    bp = (F32P * n)(*[b.ctypes.data_as(F32P) for b in B_list])
    sc = None if scales is None else _f32(scales)
    lib().oracle_merge_bf16(n, ap, bp, ranks.ctypes.data_as(I64P), _p(sc, F32P), K, N,
                            A.ctypes.data_as(U16P), B.ctypes.data_as(U16P))
    return A, B


# ------------------------------------------------------------ LoRA linear
def lora_linear_rows(X, W0, A, B, scale=1.0, bias=None, residual=None, rows=None,
                     swiglu=False, nthreads=0):
    """Y[rows] = X[rows]·W0ᵀ + scale·(X[rows]·Aᵀ)·Bᵀ (+ bias) (then SwiGLU) (+ residual).

    X: [M, K] (float32 values); W0 [N, K]; A [r, K]; B [N, r]; bias [N] or None;
    residual [M, Nout] or None.  rows: int64 indices into X (None = all rows).
    Returns float64 [len(rows), Nout].
    """
    X = _f32(X)
    W0 = _f32(W0)
    N, K = W0.shape
    r = 0 if A is None else int(np.asarray(A).shape[0])
    A = _f32(A if r else np.zeros((1, K)))
    B = _f32(B if r else np.zeros((N, 1)))
    bias = None if bias is None else _f32(bias)
    residual = None if residual is None else _f32(residual)
    if rows is None:
        rows_a = None
        nrows = X.shape[0]
    else:
        rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_a.shape[0]
    nout = N // 2 if swiglu else N
    Y = np.empty((nrows, nout), np.float64)
    if nrows == 0:
        return Y
    lib().oracle_lora_linear_rows(
        X.ctypes.data_as(F32P), X.shape[1], _p(rows_a, I64P), nrows, W0.ctypes.data_as(F32P),
        A.ctypes.data_as(F32P), B.ctypes.data_as(F32P), _p(bias, F32P), _p(residual, F32P),
        0 if residual is None else residual.shape[1], float(scale), N, K, r, int(bool(swiglu)),
        Y.ctypes.data_as(F64P), _nt(nthreads))
    return Y


def lora_linear_drows(Xd, W0, A, B, scale=1.0, nthreads=0):
    """The linear map (no bias) applied to float64 rows Xd [n, K]."""
    Xd = _f64(np.atleast_2d(Xd))
    W0 = _f32(W0)
    N, K = W0.shape
    r = 0 if A is None else int(np.asarray(A).shape[0])
    A = _f32(A if r else np.zeros((1, K)))
    B = _f32(B if r else np.zeros((N, 1)))
    Y = np.empty((Xd.shape[0], N), np.float64)
    lib().oracle_lora_linear_drows(Xd.ctypes.data_as(F64P), K, Xd.shape[0],
                                   W0.ctypes.data_as(F32P), A.ctypes.data_as(F32P),
                                   B.ctypes.data_as(F32P), float(scale), N, K, r,
                                   Y.ctypes.data_as(F64P), _nt(nthreads))
    return Y


def lora_linear_adjoint(U, W0, A, B, scale=1.0, bias=None):
    """The LoRA linear's adjoint applied to k column vectors U [N, k]:
    G = W0ᵀ·U + scale·Aᵀ·(Bᵀ·U)  [K, k]  and  c = biasᵀ·U  [k]  (zeros without bias),
    so that for every row x:  (x·W0ᵀ + scale·(x·Aᵀ)·Bᵀ + bias)·U = x·G + c.
    Freivalds' identity with the projection on the output columns: checking one
    row of a full-size output then costs K multiply-adds instead of K·N.  Steps
    are float64 matrix products of the given factors (no rounding of its own).
    Pinned against lora_linear_rows(X)·U on random cases (tests/test_checks.py)."""
    U = _f64(U)
    W0 = _f64(W0)
    G = W0.T @ U
    if A is not None and np.asarray(A).size:
        G = G + float(scale) * (_f64(A).T @ (_f64(B).T @ U))
    c = _f64(bias) @ U if bias is not None else np.zeros(U.shape[1])
    return G, c


def embed_rows(z, E):
    """x = z·Eᵀ for fp32 latent rows z [T, C] and E [D, C]; float64 [T, D]."""
    z = _f32(np.atleast_2d(z))
    E = _f32(E)
    T, C = z.shape
    D = E.shape[0]
    x = np.empty((T, D), np.float64)
    lib().oracle_embed_rows(z.ctypes.data_as(F32P), T, E.ctypes.data_as(F32P), C, D,
                            x.ctypes.data_as(F64P))
    return x


def head_rows(H, P):
    """v = H·Pᵀ for P [C, D] and rows H [T, ldh], ldh >= D, of which only the
    first D columns are read (row stride ldh, as a strided activation); float64 [T, C]."""
    H = _f32(np.atleast_2d(H))
    P = _f32(P)
    T, ldh = H.shape
    C, D = P.shape
    if ldh < D:
        raise ValueError("H rows are shorter than P's")
    v = np.empty((T, C), np.float64)
    lib().oracle_head_rows(H.ctypes.data_as(F32P), T, ldh, P.ctypes.data_as(F32P), C, D,
                           v.ctypes.data_as(F64P))
    return v


# ------------------------------------------------------------ sampler
SIGMAS = (0.909, 0.857, 0.667, 0.0)   # [EN] "Three steps instead of dozens", schedule


# ---- in-context (IC) sampler routes ([IC] section "三步接着放大的草稿画,八步从噪声重画")
# The pages name an 8-step noise table with video shift 12 but print no formula.
# Reading: the usual time-shifted flow-matching table sigma = s·t / (1 + (s-1)·t)
# on t = 1, 7/8, ..., 0, which reproduces the pages' up4 start 0.923 at t = 1/2.
# up3's printed start 0.835 is not a point of that table (its last-three start is
# 0.878): the route mixes to the printed 0.835 and then takes the table's last
# three targets.  Parity unpinned beyond the 0.923 point and the end points.
IC_TABLE_STEPS = 8
IC_VIDEO_SHIFT = 12.0
IC_ROUTE_START = {"up3": (0.835, 3), "up4": (0.923, 4), "hf8": (1.0, 8)}
REFERENCE_ROW_SIGMA = 0.001


def shifted_table(steps=IC_TABLE_STEPS, shift=IC_VIDEO_SHIFT):
    """sigma_k = shift·t_k / (1 + (shift - 1)·t_k), t_k = 1 - k/steps, k = 0..steps (fp64)."""
    out = []
    for k in range(steps + 1):
        t = 1.0 - k / steps
        out.append(shift * t / (1.0 + (shift - 1.0) * t))
    return out


def ic_route(route):
    """sigma sequence of an IC route: the printed start, then the last n table targets."""
    start, n = IC_ROUTE_START[route]
    table = shifted_table()
    return [start] + table[len(table) - n:]


def renoise(u, eps, sigma):
    u = _f32(u)
    eps = _f32(eps)
    z = np.empty(u.shape, np.float64)
    lib().oracle_renoise(u.ctypes.data_as(F32P), eps.ctypes.data_as(F32P), float(sigma),
                         z.ctypes.data_as(F64P), u.size)
    return z


def euler_step(z, v, sigma, sigma_next):
    z = _f64(z).copy()
    v = _f64(v)
    lib().oracle_euler_step(z.ctypes.data_as(F64P), v.ctypes.data_as(F64P), float(sigma),
                            float(sigma_next), z.size)
    return z


def sampler_exact_velocity(x0, eps, sigmas=SIGMAS):
    """Renoise then Euler with v = eps - x0; returns [len(sigmas), *x0.shape]."""
    x0 = _f32(x0)
    eps = _f32(eps)
    s = _f64(sigmas)
    z = np.empty((len(s),) + x0.shape, np.float64)
    lib().oracle_sampler_exact_velocity(x0.ctypes.data_as(F32P), eps.ctypes.data_as(F32P),
                                        s.ctypes.data_as(F64P), len(s), z.ctypes.data_as(F64P),
                                        x0.size)
    return z


# ------------------------------------------------------------ stand-in
def _layers(layers, keep):
    arr = (LoraLayer * 4)()
    for i, L in enumerate(layers):
        W0 = _f32(L["W0"])
        N, K = W0.shape
        r = int(np.asarray(L["A"]).shape[0]) if L.get("A") is not None else 0
        A = _f32(L["A"] if r else np.zeros((1, K)))
        B = _f32(L["B"] if r else np.zeros((N, 1)))
        bias = None if L.get("bias") is None else _f32(L["bias"])
        keep += [W0, A, B, bias]
        arr[i] = LoraLayer(W0.ctypes.data_as(F32P), A.ctypes.data_as(F32P),
                           B.ctypes.data_as(F32P), _p(bias, F32P), N, K, r,
                           float(L.get("scale", 1.0)))
    return arr


def standin_refine(x0, eps, E, P, layers, sigmas=SIGMAS, nthreads=0):
    """Run renoise + Euler steps of the velocity stand-in on token rows.

    x0, eps: [T, C]; E [D, C]; P [C, D]; layers: 4 dicts (W0, A, B, bias, scale)
    for qkv (3D x D), o (D x D), gate/up (2F x D), down (D x F).
    Returns (z_hist [nsig, T, C], v_hist [nsig-1, T, C]).
    """
    x0 = _f32(x0)
    eps = _f32(eps)
    E = _f32(E)
    P = _f32(P)
    T, C = x0.shape
    D = E.shape[0]
    F = _f32(layers[3]["W0"]).shape[1]
    s = _f64(sigmas)
    keep = []
    arr = _layers(layers, keep)
    z = np.empty((len(s), T, C), np.float64)
    v = np.empty((len(s) - 1, T, C), np.float64)
    lib().oracle_standin_refine(x0.ctypes.data_as(F32P), eps.ctypes.data_as(F32P), T,
                                s.ctypes.data_as(F64P), len(s), E.ctypes.data_as(F32P),
                                P.ctypes.data_as(F32P), C, D, F, arr, z.ctypes.data_as(F64P),
                                v.ctypes.data_as(F64P), _nt(nthreads))
    return z, v


def standin_velocity(z, E, P, layers):
    """The stand-in's velocity for float64 latent rows z [T, C]."""
    z = _f64(np.atleast_2d(z))
    E = _f32(E)
    P = _f32(P)
    T, C = z.shape
    D = E.shape[0]
    F = _f32(layers[3]["W0"]).shape[1]
    keep = []
    arr = _layers(layers, keep)
    v = np.empty((T, C), np.float64)
    lib().oracle_standin_velocity(z.ctypes.data_as(F64P), T, E.ctypes.data_as(F32P),
                                  P.ctypes.data_as(F32P), C, D, F, arr, v.ctypes.data_as(F64P))
    return v
