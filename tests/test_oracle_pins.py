"""Pins of the oracle's stand-in projections and of the MXFP8 stand-in data flow
against computations that share nothing with them.

* oracle.embed_rows / oracle.head_rows (the reference of the embed, head and
  head+Euler GPU tests): exact rational sums (fractions.Fraction) on tiny
  shapes, channel counts 1, 24, 32 and 70, and head rows read with a row stride
  wider than D whose skipped columns hold non-finite values; numpy float64
  products at the stand-in's width.
* oracle.mx.standin_velocity_mx: one token taken through the MXFP8 data flow
  stage by stage with an independent quantizer (E4M3 through torch's
  float8_e4m3fn cast after a clamp to +-448, E8M0 scale from math.frexp of the
  block maximum, bf16 through torch's bfloat16 cast, sums in Fractions), each
  stage compared with the oracle's own intermediate.  Each quantization point
  is then shown to matter: dropping or moving it in the independent flow moves
  the velocity by far more than the comparison tolerance, so a misplaced
  rounding in the oracle would fail this test.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import mx


def _bf16(x):
    """bf16-representable float32 values (torch's nearest-even cast)."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _exact_rows(A, B):
    """Exact A·Bᵀ with Fractions, as float64 (one rounding at the end)."""
    out = np.empty((A.shape[0], B.shape[0]))
    for i in range(A.shape[0]):
        for j in range(B.shape[0]):
            s = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(A[i], B[j])),
                    Fraction(0))
            out[i, j] = float(s)
    return out


@pytest.mark.parametrize("C", [1, 24, 32, 70])
def test_embed_rows_exact(C):
    rng = np.random.default_rng(100 + C)
    T, D = 3, 16
    z = (rng.standard_normal((T, C)) * np.exp(rng.standard_normal((T, C)))).astype(np.float32)
    E = _bf16(rng.standard_normal((D, C)) / math.sqrt(C))
    got = oracle.embed_rows(z, E)
    ref = _exact_rows(z.astype(np.float64), E.astype(np.float64))
    bound = np.abs(z.astype(np.float64)) @ np.abs(E.astype(np.float64)).T
    assert np.all(np.abs(got - ref) <= 1e-15 * C * bound + 1e-300)


@pytest.mark.parametrize("C,ldh_extra", [(1, 0), (24, 0), (24, 8), (32, 40), (3, 64)])
def test_head_rows_exact_and_strided(C, ldh_extra):
    rng = np.random.default_rng(200 + C + ldh_extra)
    T, D = 4, 64
    H = np.full((T, D + ldh_extra), np.nan, np.float32)
    H[:, D:] = np.where(rng.random((T, ldh_extra)) < 0.5, np.inf, np.nan)
    H[:, :D] = _bf16(rng.standard_normal((T, D)) * 3.0)
    P = _bf16(rng.standard_normal((C, D)) / math.sqrt(D))
    got = oracle.head_rows(H, P)
    assert np.all(np.isfinite(got)), "read past D in a strided row"
    ref = _exact_rows(H[:, :D].astype(np.float64), P.astype(np.float64))
    bound = np.abs(H[:, :D].astype(np.float64)) @ np.abs(P.astype(np.float64)).T
    assert np.all(np.abs(got - ref) <= 1e-15 * D * bound)


def test_embed_and_head_at_standin_width_against_numpy():
    rng = np.random.default_rng(7)
    T, C, D = 9, 24, 3072
    z = rng.standard_normal((T, C)).astype(np.float32)
    E = _bf16(rng.standard_normal((D, C)) / math.sqrt(C))
    x = oracle.embed_rows(z, E)
    np.testing.assert_allclose(x, z.astype(np.float64) @ E.astype(np.float64).T,
                               rtol=1e-12, atol=1e-12)
    H = _bf16(rng.standard_normal((T, D + 64)))
    P = _bf16(rng.standard_normal((C, D)) / math.sqrt(D))
    v = oracle.head_rows(H, P)
    np.testing.assert_allclose(v, H[:, :D].astype(np.float64) @ P.astype(np.float64).T,
                               rtol=1e-12, atol=1e-12)


def test_head_rows_rejects_short_rows():
    with pytest.raises(ValueError):
        oracle.head_rows(np.zeros((2, 8), np.float32), np.zeros((1, 16), np.float32))


# ------------------------------------------------------- MXFP8 stand-in, one token
def _ind_bf16(v):
    """bf16 rounding of float32(v) by torch's cast (the data flow rounds fp32 values)."""
    t = torch.tensor(np.asarray(v, np.float64), dtype=torch.float32)
    return t.to(torch.bfloat16).double().numpy()


def _ind_mx(row):
    """Dequantized MXFP8 of one row, independently: per 32-block, scale
    2^(floor(log2 amax) - 8) from math.frexp, elements through torch's
    float8_e4m3fn cast of the clamped quotient."""
    row = np.asarray(row, np.float64)
    out = np.empty_like(row)
    for b in range(0, row.size, 32):
        blk = row[b:b + 32]
        amax = float(np.max(np.abs(blk)))
        e = -127 if amax == 0.0 else max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
        y = np.clip(np.ldexp(blk, -e), -448.0, 448.0)
        q = torch.tensor(y, dtype=torch.float64).to(torch.float8_e4m3fn).double().numpy()
        out[b:b + 32] = np.ldexp(q, e)
    return out


def _fdot(a, b):
    return float(sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, b)),
                     Fraction(0)))


def _ind_linear(x, L, *, quant_x=True, quant_t=True, round_t=True):
    """One MXFP8 LoRA linear for one token: y = q(x)·q(W0)ᵀ + q(bf16(s·q(x)·q(A)ᵀ))·q(B)ᵀ."""
    qm = lambda M: np.stack([_ind_mx(r) for r in M])
    xq = _ind_mx(x) if quant_x else np.asarray(x, np.float64)
    W0, A, B = qm(L["W0"]), qm(L["A"]), qm(L["B"])
    t = np.array([L["scale"] * _fdot(xq, A[j]) for j in range(A.shape[0])])
    if round_t:
        t = _ind_bf16(t)
    tq = _ind_mx(t) if quant_t else t
    return np.array([_fdot(xq, W0[n]) + _fdot(tq, B[n]) for n in range(W0.shape[0])])


def _ind_token(z, E, P, layers, skip=None):
    """The stand-in for one token with every rounding point written out; `skip`
    names one point to leave out (to show that each one is observable)."""
    D = E.shape[0]
    F = layers[3]["W0"].shape[1]
    r = lambda name, v: v if skip == name else _ind_bf16(v)
    x = r("x", np.array([_fdot(z, E[n]) for n in range(D)]))
    qkv = r("qkv", _ind_linear(x, layers[0], quant_x=skip != "quant_x"))
    h1 = r("h1", _ind_linear(qkv[2 * D:3 * D], layers[1], quant_t=skip != "quant_t") + x)
    y = _ind_linear(h1, layers[2], round_t=skip != "round_t")
    gate, up = y[:F], y[F:]
    g = r("g", np.array([a / (1.0 + math.exp(-a)) * b for a, b in zip(gate, up)]))
    h2 = r("h2", _ind_linear(g, layers[3]) + h1)
    v = np.array([_fdot(h2, P[c]) for c in range(P.shape[0])])
    return dict(x=x, qkv=qkv, h1=h1, g=g, h2=h2, v=v)


def _token_fixture():
    rng = np.random.default_rng(31)
    C, D, F, rank = 4, 32, 32, 32
    bf = mx.bf16_round_np
    layers = []
    for K, N in [(D, 3 * D), (D, D), (D, 2 * F), (F, D)]:
        layers.append({"W0": bf(rng.standard_normal((N, K)) * 0.3),
                       "A": bf(rng.standard_normal((rank, K)) / math.sqrt(K)),
                       "B": bf(rng.standard_normal((N, rank)) * 0.2), "scale": 0.75})
    E = bf(rng.standard_normal((D, C)))
    P = bf(rng.standard_normal((C, D)) * 0.1)
    z = rng.standard_normal(C)
    return z, E, P, layers


def test_mx_standin_token_stage_by_stage():
    z, E, P, layers = _token_fixture()
    tr = {}
    v = mx.standin_velocity_mx(z[None, :], E, P, mx.standin_mx_weights(layers), trace=tr)[0]
    ref = _ind_token(z, E, P, layers)
    for name in ("x", "qkv", "h1", "g", "h2"):
        got = tr[name][0]
        # bf16 activations: both sides round the same fp64-accurate value, so they
        # agree exactly except where that value lies within fp rounding of a tie
        mism = np.mean(got != ref[name])
        assert mism <= 0.02, (name, mism)
    np.testing.assert_allclose(v, ref["v"], rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("point", ["x", "qkv", "quant_x", "quant_t", "round_t", "h1", "g", "h2"])
def test_mx_standin_each_rounding_point_is_observable(point):
    """Leaving out any one quantization or rounding point moves the token's
    velocity by far more than the tolerance of the stage-by-stage test, so the
    oracle could not misplace one and still pass it."""
    z, E, P, layers = _token_fixture()
    full = _ind_token(z, E, P, layers)["v"]
    moved = _ind_token(z, E, P, layers, skip=point)["v"]
    rel = np.linalg.norm(moved - full) / np.linalg.norm(full)
    assert rel > 1e-4, (point, rel)
