"""The oracle's LoRA linear against exact arithmetic and an independent library.

Pins for oracle.lora_linear_rows (a2-a4):
  * small-integer inputs: every product and partial sum is an exact integer in
    fp64, so the oracle must equal the exact result bit for bit;
  * dyadic (bf16-like) inputs: exact rational arithmetic with Fraction, within
    the fp64 summation bound;
  * numpy float64 matmul (a library routine) on the tiny workload.
A dropped term, a wrong index or a transposed operand fails all three.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from few_step_diffusion_amd import inputs


def exact_lora(X, W0, A, B, s, bias=None):
    """Y = X·W0ᵀ + s·(X·Aᵀ)·Bᵀ + bias in exact rationals (pure Python, tiny shapes)."""
    M, K = X.shape
    N = W0.shape[0]
    r = 0 if A is None else A.shape[0]
    Xf = [[Fraction(float(v)) for v in row] for row in X]
    out = []
    for m in range(M):
        t = [sum((Xf[m][k] * Fraction(float(A[j, k])) for k in range(K)), Fraction(0))
             for j in range(r)]
        row = []
        for n in range(N):
            y = sum((Xf[m][k] * Fraction(float(W0[n, k])) for k in range(K)), Fraction(0))
            y += Fraction(s) * sum((t[j] * Fraction(float(B[n, j])) for j in range(r)), Fraction(0))
            if bias is not None:
                y += Fraction(float(bias[n]))
            row.append(y)
        out.append(row)
    return out


@pytest.mark.parametrize("M,N,K,r,s", [(5, 7, 9, 0, 1.0), (6, 8, 24, 3, 1.0), (24, 16, 12, 6, 0.5),
                                       (3, 24, 20, 6, 2.0), (1, 1, 1, 1, 1.0)])
def test_integer_inputs_exact(M, N, K, r, s):
    g = np.random.Generator(np.random.PCG64(7 + M * 31 + N))
    X = g.integers(-8, 9, (M, K)).astype(np.float32)
    W0 = g.integers(-8, 9, (N, K)).astype(np.float32)
    A = g.integers(-8, 9, (r, K)).astype(np.float32) if r else None
    B = g.integers(-8, 9, (N, r)).astype(np.float32) if r else None
    bias = g.integers(-8, 9, N).astype(np.float32)
    Y = oracle.lora_linear_rows(X, W0, A, B, scale=s, bias=bias)
    E = exact_lora(X, W0, A, B, s, bias)
    for m in range(M):
        for n in range(N):
            assert Fraction(Y[m, n]) == E[m][n], (m, n)


def _dyadic(g, shape, lo=-6, hi=2):
    """Random bf16-representable values: 8-bit significand, exponent in [lo, hi]."""
    mant = g.integers(128, 256, shape) * g.choice([-1, 1], shape)
    exp = g.integers(lo, hi + 1, shape)
    return (mant * np.exp2(exp - 7.0)).astype(np.float32)


@pytest.mark.parametrize("M,N,K,r", [(4, 6, 16, 3), (8, 5, 24, 6), (2, 24, 24, 6)])
def test_dyadic_inputs_within_fp64_bound(M, N, K, r):
    g = np.random.Generator(np.random.PCG64(100 + M + N + K))
    X, W0 = _dyadic(g, (M, K)), _dyadic(g, (N, K))
    A, B = _dyadic(g, (r, K)), _dyadic(g, (N, r))
    s = 0.75
    Y = oracle.lora_linear_rows(X, W0, A, B, scale=s)
    E = exact_lora(X, W0, A, B, s)
    # fp64 bound: (terms) * eps * sum of |terms|, terms = K + r*(K+1) products
    absX = np.abs(X.astype(np.float64))
    mag = absX @ np.abs(W0.T.astype(np.float64)) + \
        abs(s) * (absX @ np.abs(A.T.astype(np.float64))) @ np.abs(B.T.astype(np.float64))
    nterms = K + r * (K + 1)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(Y[m, n]) - E[m][n])
            assert float(err) <= 2 * nterms * 2.0 ** -53 * mag[m, n], (m, n, float(err))


def test_numpy_float64_cross_check_tiny_workload():
    wl = inputs.WORKLOADS[0]
    _, K, N, _ = wl.linears[0]
    M = wl.tokens
    X = inputs.activations(0, M, K).float().numpy()
    W0 = inputs.base_weight(0, K, N).float().numpy()
    A_l, B_l = inputs.adapters(0, K, N)
    Ab, Bb = oracle.merge_bf16([a.numpy() for a in A_l], [b.numpy() for b in B_l])
    A = oracle.bf16_value(Ab)
    B = oracle.bf16_value(Bb)
    bias = inputs.bias(0, N).numpy()
    Y = oracle.lora_linear_rows(X, W0, A, B, scale=1.0, bias=bias)
    X64 = X.astype(np.float64)
    ref = X64 @ W0.T.astype(np.float64) + (X64 @ A.T.astype(np.float64)) @ B.T.astype(np.float64) \
        + bias.astype(np.float64)
    rel = np.abs(Y - ref).max() / np.abs(ref).max()
    assert rel <= 1e-12, rel


def test_sampled_rows_match_full_rows():
    g = np.random.Generator(np.random.PCG64(3))
    X = _dyadic(g, (40, 16))
    W0, A, B = _dyadic(g, (8, 16)), _dyadic(g, (4, 16)), _dyadic(g, (8, 4))
    full = oracle.lora_linear_rows(X, W0, A, B)
    rows = np.array([39, 0, 17, 17, 5], dtype=np.int64)
    part = oracle.lora_linear_rows(X, W0, A, B, rows=rows)
    assert np.array_equal(part, full[rows])


def test_drows_is_the_same_linear_map():
    g = np.random.Generator(np.random.PCG64(4))
    X = _dyadic(g, (6, 16))
    W0, A, B = _dyadic(g, (8, 16)), _dyadic(g, (4, 16)), _dyadic(g, (8, 4))
    a = oracle.lora_linear_rows(X, W0, A, B, scale=0.5)
    b = oracle.lora_linear_drows(X.astype(np.float64), W0, A, B, scale=0.5)
    assert np.array_equal(a, b)
