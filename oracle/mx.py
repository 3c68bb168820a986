"""fp64 reference of MXFP8 (E4M3 elements, E8M0 block scales) — TEST INFRASTRUCTURE ONLY.

The pages replace the refiner's bf16 linears by MXFP8 linears (FP8 GEMMs whose
operands are quantized again at every stage) and fuse SwiGLU with a one-pass
activation quantizer
([EN] "Open-H3-Regenerate-2K: High-Resolution Video Refinement with Few-Step
Diffusion", section "Where the 3.9x speedup comes from", inference-configuration
table).  They give no block size, scale rule or rounding; the reading taken is the
OCP "Microscaling Formats (MX) Specification" v1.0, MXFP8 E4M3:
  * blocks of 32 consecutive elements along the reduction (K) dimension;
  * shared scale X = 2^(floor(log2(amax)) - 8), 8 being E4M3's largest exponent,
    stored as E8M0 (exponent + 127; an all-zero block gets the smallest, 2^-127);
  * elements x/X rounded to nearest-even in E4M3 (bias 7, 3 mantissa bits,
    subnormals down to 2^-9), magnitudes past the largest finite value 448
    saturated to 448.
Everything here is plain numpy float64, element by element where it matters.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest power of two below E4M3_MAX
E4M3_EMIN = -6         # smallest normal exponent; the quantum below it is 2^-9
MX_BLOCK = 32


def e4m3_round(y: float) -> float:
    """Nearest-even E4M3 value of y, saturated to +-448 (y finite)."""
    a = abs(y)
    if a == 0.0:
        return 0.0 * y
    m, ex = math.frexp(a)              # a = m·2^ex, 0.5 <= m < 1 (exact floor(log2))
    e = max(ex - 1, E4M3_EMIN)
    q = math.ldexp(1.0, e - 3)         # spacing of E4M3 values in [2^e, 2^(e+1))
    k = a / q                          # exact: q is a power of two
    r = math.floor(k)
    frac = k - r
    if frac > 0.5 or (frac == 0.5 and r % 2 == 1):
        r += 1
    v = min(r * q, E4M3_MAX)
    return math.copysign(v, y)


def e4m3_bits(v: float) -> int:
    """Byte of an E4M3-representable value v (sign, 4-bit exponent with bias 7, 3-bit mantissa)."""
    s = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a == 0.0:
        return s
    m, ex = math.frexp(a)
    e = ex - 1
    if e < E4M3_EMIN:                  # subnormal: a = mant·2^-9
        mant = a / math.ldexp(1.0, E4M3_EMIN - 3)
        assert mant == int(mant) and 0 < mant < 8
        return s | int(mant)
    mant = (a / math.ldexp(1.0, e) - 1.0) * 8.0
    assert mant == int(mant) and 0 <= mant < 8 and e <= E4M3_EMAX
    return s | ((e + 7) << 3) | int(mant)


def e4m3_value(b: int) -> float:
    """Value of an E4M3 byte (0x7f / 0xff are NaN and never produced here)."""
    s = -1.0 if b & 0x80 else 1.0
    e = (b >> 3) & 0xF
    m = b & 7
    if e == 0:
        return s * math.ldexp(m / 8.0, E4M3_EMIN)
    return s * math.ldexp(1.0 + m / 8.0, e - 7)


def block_exponent(block) -> int:
    """Shared exponent of one block: floor(log2(amax)) - 8, clamped to E8M0's [-127, 127]."""
    amax = max(abs(float(x)) for x in block)
    if amax == 0.0:
        return -127
    m, ex = math.frexp(amax)
    return max(-127, min(127, (ex - 1) - E4M3_EMAX))


def quantize_rows(X, K=None):
    """MXFP8 of the rows of X (float values) along their length.

    Returns (q, s): q uint8 [rows, Kp] E4M3 bytes, Kp = K rounded up to a
    multiple of 128 (the padding holds zeros), and s uint8 [rows, Kp/32] E8M0
    bytes (padded blocks get 127, i.e. a scale of 1).
    """
    X = np.asarray(X, dtype=np.float64)
    rows, K0 = X.shape
    K = K0 if K is None else K
    Kp = (K + 127) // 128 * 128
    q = np.zeros((rows, Kp), np.uint8)
    s = np.full((rows, Kp // MX_BLOCK), 127, np.uint8)
    for i in range(rows):
        for b in range(0, K, MX_BLOCK):
            blk = X[i, b:b + MX_BLOCK]
            se = block_exponent(blk)
            s[i, b // MX_BLOCK] = se + 127
            for j, x in enumerate(blk):
                q[i, b + j] = e4m3_bits(e4m3_round(math.ldexp(float(x), -se)))
    return q, s


def dequantize_rows(q, s, K):
    """Float64 values [rows, K] of MXFP8 rows (element value times its block's scale)."""
    rows = q.shape[0]
    out = np.empty((rows, K), np.float64)
    for i in range(rows):
        for k in range(K):
            out[i, k] = math.ldexp(e4m3_value(int(q[i, k])), int(s[i, k // MX_BLOCK]) - 127)
    return out


# ------------------------------------------------------------------ array form
# The same quantizer over whole arrays, for matrices too large for the element
# loops above: every step is the scalar one (np.frexp gives the exact binade,
# np.rint rounds half to even, np.ldexp scales exactly).  Pinned to
# quantize_rows / dequantize_rows element for element by the CPU tests.
_E4M3_TABLE = np.array([e4m3_value(b) if (b & 0x7F) != 0x7F else 0.0 for b in range(256)])


def e4m3_round_np(y):
    """e4m3_round over an array (float64 in, float64 out)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, ey = np.frexp(a)                             # a = m·2^ey, 0.5 <= m < 1
    binade = np.maximum(ey.astype(np.int64) - 1, E4M3_EMIN)
    quantum = np.ldexp(1.0, binade - 3)
    v = np.minimum(np.rint(a / quantum) * quantum, E4M3_MAX)   # nearest-even, saturated
    return np.copysign(v, y)


def block_exponents_np(X):
    """block_exponent of every 32-element block of the rows of X: int64 [rows, K/32]."""
    X = np.asarray(X, dtype=np.float64)
    rows, K = X.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    amax = np.abs(X.reshape(rows, K // MX_BLOCK, MX_BLOCK)).max(axis=2)
    _, ex = np.frexp(amax)                          # amax = m·2^ex, 0.5 <= m < 1
    e = np.clip(ex.astype(np.int64) - 1 - E4M3_EMAX, -127, 127)
    return np.where(amax == 0.0, -127, e)


def e4m3_bits_np(v):
    """e4m3_bits over an array of E4M3-representable values."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ev = np.frexp(a)
    ev = ev.astype(np.int64) - 1
    normal = a >= math.ldexp(1.0, E4M3_EMIN)
    ev_n = np.where(normal, ev, 0)
    mant_n = (np.ldexp(a, -ev_n) - 1.0) * 8.0
    code_n = ((ev_n + 7) << 3) | mant_n.astype(np.int64)
    code_s = (a / math.ldexp(1.0, E4M3_EMIN - 3)).astype(np.int64)
    return (np.where(normal, code_n, code_s) | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def quantize_rows_np(X):
    """quantize_rows for K a multiple of 32, as array operations."""
    X = np.asarray(X, dtype=np.float64)
    rows, K = X.shape
    Kp = (K + 127) // 128 * 128
    e = block_exponents_np(X)
    y = np.ldexp(X, -np.repeat(e, MX_BLOCK, axis=1))   # exact: power-of-two scaling
    q = np.zeros((rows, Kp), np.uint8)
    q[:, :K] = e4m3_bits_np(e4m3_round_np(y))
    s = np.full((rows, Kp // MX_BLOCK), 127, np.uint8)
    s[:, :K // MX_BLOCK] = (e + 127).astype(np.uint8)
    return q, s


def dequantize_rows_np(q, s, K):
    """dequantize_rows as array operations."""
    q = np.asarray(q)[:, :K]
    sc = np.asarray(s, dtype=np.int64)[:, np.arange(K) // MX_BLOCK] - 127
    return np.ldexp(_E4M3_TABLE[q], sc)


# ------------------------------------------------------- MXFP8 stand-in velocity
# The velocity stand-in of the refine loop (see standin_velocity in this
# package) with its four linears run as MXFP8 GEMMs, at the quantization points
# the pages' MXFP8 inference path implies: activations live in bf16 between
# operations and are quantized at each linear's input, the LoRA down output T
# is rounded to bf16 and quantized before the up projection, SwiGLU's bf16
# output is quantized for the down projection, and the weights (W0, A, B) are
# quantized once from their bf16 values.  Sums are exact (fp64 matmul of the
# dequantized values); every bf16 rounding is nearest-even.
def bf16_round_np(x):
    """Nearest-even bfloat16 value of float32(x), as float64 (x finite)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    r = (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def mx_values(X):
    """Dequantized MXFP8 of the rows of X ([rows, K], K a multiple of 32)."""
    X = np.asarray(X, dtype=np.float64)
    q, s = quantize_rows_np(X)
    return dequantize_rows_np(q, s, X.shape[1])


def standin_mx_weights(layers):
    """(W0, A, B) of each layer as dequantized MXFP8 (from their bf16 values) plus scale."""
    out = []
    for L in layers:
        out.append({"W0": mx_values(L["W0"]), "A": mx_values(L["A"]), "B": mx_values(L["B"]),
                    "scale": float(L.get("scale", 1.0))})
    return out


def _mx_linear(Xb, L):
    Xd = mx_values(Xb)
    T = bf16_round_np(L["scale"] * (Xd @ L["A"].T))
    return Xd @ L["W0"].T + mx_values(T) @ L["B"].T


def standin_velocity_mx(z, E, P, wq, trace=None):
    """Velocity of float64 latent rows z [T, C]; E [D, C], P [C, D]; wq from
    standin_mx_weights (qkv, o, gate/up, down).  Returns float64 [T, C].
    trace: a dict to receive the bf16 activations between the operations
    (x, qkv, h1, g, h2) for stage-by-stage checks."""
    z = np.asarray(z, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    D = E.shape[0]
    F = wq[3]["W0"].shape[1]
    h = bf16_round_np(z @ E.T)
    x = h
    qkv = bf16_round_np(_mx_linear(h, wq[0]))
    h = bf16_round_np(_mx_linear(qkv[:, 2 * D:3 * D], wq[1]) + h)
    h1 = h
    y = _mx_linear(h, wq[2])
    gate, up = y[:, :F], y[:, F:]
    g = bf16_round_np(gate / (1.0 + np.exp(-gate)) * up)
    h = bf16_round_np(_mx_linear(g, wq[3]) + h)
    if trace is not None:
        trace.update(x=x, qkv=qkv, h1=h1, g=g, h2=h)
    return h @ P.T


def standin_refine_mx(x0, eps, E, P, wq, sigmas):
    """Renoise at sigmas[0], then one MXFP8 stand-in velocity and Euler step per
    sigma pair (fp64 latent).  Returns the final latent [T, C]."""
    from . import euler_step, renoise
    z = renoise(x0, eps, sigmas[0])
    for k in range(len(sigmas) - 1):
        z = euler_step(z, standin_velocity_mx(z, E, P, wq), sigmas[k], sigmas[k + 1])
    return z
