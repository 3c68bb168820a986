"""Checks of full-size GPU outputs against the oracle (test infrastructure).

row_projection_check: every row of a LoRA-linear output Y = X·W0ᵀ +
s·(X·Aᵀ)·Bᵀ + bias (+ residual) is checked through k random column projections
(Freivalds' identity on the output columns).  The oracle supplies the adjoint
G = W0ᵀ·U + s·Aᵀ·(Bᵀ·U) and c = biasᵀ·U once; per row the expected projections
are X_i·G + c (+ R_i·U), K multiply-adds, so every one of 532,800 rows is
checked without a per-row K·N product.  The statistic per row is

    e_i = ‖Y_i·U − (X_i·G + c + R_i·U)‖₂ / (‖Y_i‖₂·√k),

an estimate of the row's relative L2 error ‖ΔY_i‖₂/‖Y_i‖₂ (for Gaussian U,
E‖d·U‖² = k‖d‖²), gated like a directly compared row.  A defect confined to one
row is not diluted by other rows; the CPU tests plant a lost rank-64 adapter
in one row and show the check fails on it.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from oracle import metrics


def projection(N, K, W0, A, B, scale=1.0, bias=None, k=16, seed=0):
    """(U [N, k], G [K, k], c [k]) for the linear with factors W0, A, B."""
    g = np.random.Generator(np.random.PCG64(seed))
    U = g.standard_normal((N, k))
    G, c = oracle.lora_linear_adjoint(U, W0, A, B, scale=scale, bias=bias)
    return U, G, c


def row_projection_errors(X, Y, U, G, c, residual=None, chunk=32768):
    """e_i for every row (float64 numpy array), computed in float64 on Y's device."""
    dev = Y.device
    Ut = torch.from_numpy(np.ascontiguousarray(U)).to(dev)
    Gt = torch.from_numpy(np.ascontiguousarray(G)).to(dev)
    ct = torch.from_numpy(np.ascontiguousarray(c)).to(dev)
    k = U.shape[1]
    out = []
    for r0 in range(0, Y.shape[0], chunk):
        r1 = min(Y.shape[0], r0 + chunk)
        Yd = Y[r0:r1].double()
        got = Yd @ Ut
        exp = X[r0:r1].double() @ Gt + ct
        if residual is not None:
            exp = exp + residual[r0:r1].double() @ Ut
        num = torch.linalg.vector_norm(got - exp, dim=1)
        den = torch.linalg.vector_norm(Yd, dim=1) * math.sqrt(k)
        e = torch.where(den > 0, num / den.clamp_min(1e-300),
                        torch.where(num > 0, torch.full_like(num, float("inf")), num))
        e = torch.where(torch.isfinite(Yd).all(dim=1), e, torch.full_like(e, float("inf")))
        out.append(e.cpu().numpy())
    return np.concatenate(out) if out else np.zeros(0)


def row_projection_check(X, Y, U, G, c, residual=None, tol=metrics.GEMM_TOL):
    """(ok, max e_i, worst row)."""
    e = row_projection_errors(X, Y, U, G, c, residual)
    worst = int(np.argmax(e)) if e.size else -1
    emax = float(e[worst]) if e.size else 0.0
    return emax <= tol, emax, worst
