"""Tolerance metrics that compare a computed result with the oracle.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).

bf16 GEMM outputs (per row of Y):
  rel_l2   = ‖ΔY‖₂ / ‖Y_ref‖₂
  rel_max  = max|ΔY| / max|Y_ref|
Both are reduced with max over rows and gated at 2e-2.  A legitimately
rounded bf16 result sits near 2e-3 and 4e-3 respectively; losing the rank-64
adapter of the merged LoRA pushes both above 8e-2 (tests/test_metrics.py).

fp32 sampler outputs (per token, the C-channel latent vector):
  rel_tok  = ‖Δz‖₂ / ‖z_ref‖₂, max over tokens, gated at 1e-5.
"""
from __future__ import annotations

import numpy as np

GEMM_TOL = 2e-2
SAMPLER_TOL = 1e-5


def row_errors(Y, Y_ref):
    """Return (max over rows of rel_l2, max over rows of rel_max)."""
    Y = np.asarray(Y, dtype=np.float64)
    Y_ref = np.asarray(Y_ref, dtype=np.float64)
    if Y.shape != Y_ref.shape:
        raise ValueError(f"shape mismatch {Y.shape} vs {Y_ref.shape}")
    if Y.size == 0:
        return 0.0, 0.0
    if not np.all(np.isfinite(Y)):
        return float("inf"), float("inf")
    d = Y - Y_ref
    den_l2 = np.linalg.norm(Y_ref, axis=1)
    den_mx = np.max(np.abs(Y_ref), axis=1)
    tiny = np.finfo(np.float64).tiny
    rel_l2 = np.linalg.norm(d, axis=1) / np.maximum(den_l2, tiny)
    rel_mx = np.max(np.abs(d), axis=1) / np.maximum(den_mx, tiny)
    return float(rel_l2.max()), float(rel_mx.max())


def gemm_ok(Y, Y_ref, tol=GEMM_TOL):
    a, b = row_errors(Y, Y_ref)
    return a <= tol and b <= tol, (a, b)


def token_error(z, z_ref):
    """Max over tokens (rows) of ‖Δz‖₂/‖z_ref‖₂."""
    z = np.asarray(z, dtype=np.float64)
    z_ref = np.asarray(z_ref, dtype=np.float64)
    if z.shape != z_ref.shape:
        raise ValueError(f"shape mismatch {z.shape} vs {z_ref.shape}")
    if z.size == 0:
        return 0.0
    if not np.all(np.isfinite(z)):
        return float("inf")
    z = z.reshape(-1, z.shape[-1])
    z_ref = z_ref.reshape(-1, z_ref.shape[-1])
    den = np.maximum(np.linalg.norm(z_ref, axis=1), np.finfo(np.float64).tiny)
    return float((np.linalg.norm(z - z_ref, axis=1) / den).max())
