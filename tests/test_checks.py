"""CPU tests of the full-size checker (tests/checks.py) and of the oracle's
adjoint that feeds it: the identity itself, the legitimate level of a
bf16-rounded output, and a planted one-row defect (the rank-64 adapter lost in
a single row) that the check must catch while a tile-projected check of the
same output would not."""
import numpy as np
import torch

import oracle
from oracle import metrics
from few_step_diffusion_amd import inputs

import checks


def _layer(K=1024, N=1024, seed=0):
    W0 = inputs.base_weight(seed, K, N).float().numpy()
    A_l, B_l = inputs.adapters(seed, K, N)
    Ab, Bb = oracle.merge_bf16([a.numpy() for a in A_l], [b.numpy() for b in B_l])
    A = oracle.bf16_value(Ab).reshape(Ab.shape).astype(np.float64)
    B = oracle.bf16_value(Bb).reshape(Bb.shape).astype(np.float64)
    return W0, A, B


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def test_adjoint_identity_against_the_rows():
    rng = np.random.default_rng(5)
    M, K, N, r = 40, 96, 80, 24
    X = _bf16(rng.standard_normal((M, K))).astype(np.float32)
    W0 = _bf16(rng.standard_normal((N, K)) * 0.1).astype(np.float32)
    A = _bf16(rng.standard_normal((r, K)) * 0.1).astype(np.float32)
    B = _bf16(rng.standard_normal((N, r)) * 0.1).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    U = rng.standard_normal((N, 7))
    for scale, b in ((1.0, None), (0.37, bias)):
        G, c = oracle.lora_linear_adjoint(U, W0, A, B, scale=scale, bias=b)
        lhs = X.astype(np.float64) @ G + c
        rhs = oracle.lora_linear_rows(X, W0, A, B, scale=scale, bias=b) @ U
        np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-11)
    # no LoRA term
    G, c = oracle.lora_linear_adjoint(U, W0, None, None)
    np.testing.assert_allclose(X.astype(np.float64) @ G,
                               oracle.lora_linear_rows(X, W0, None, None) @ U, rtol=1e-11,
                               atol=1e-11)


def _simulated_gpu_output(X, W0, A, B, drop_rank64_row=None):
    """The bf16 path's rounding: T = bf16(X·Aᵀ), Y = bf16(X·W0ᵀ + T·Bᵀ); one row
    optionally computed with the last (rank-64) adapter left out."""
    Xd = X.astype(np.float64)
    T = _bf16(Xd @ A.T)
    Y = Xd @ W0.T.astype(np.float64) + T @ B.T
    if drop_rank64_row is not None:
        i = drop_rank64_row
        Y[i] = Xd[i] @ W0.T.astype(np.float64) + T[i, :512] @ B[:, :512].T
    return _bf16(Y)


def test_row_projection_passes_legit_rounding_and_catches_one_lost_adapter_row():
    M, K, N = 300, 1024, 1024
    W0, A, B = _layer(K, N)
    X = inputs.activations(0, M, K).float().numpy()
    U, G, c = checks.projection(N, K, W0, A, B, k=16, seed=1)
    Xt = torch.from_numpy(X)
    clean = torch.from_numpy(_simulated_gpu_output(X, W0, A, B))
    ok, emax, worst = checks.row_projection_check(Xt, clean, U, G, c)
    assert ok and emax < 5e-3, emax
    # the row-level truth, for the planted row, is far above the gate
    bad_row = 137
    bad = torch.from_numpy(_simulated_gpu_output(X, W0, A, B, drop_rank64_row=bad_row))
    ref = oracle.lora_linear_rows(X[bad_row:bad_row + 1], W0, A, B)
    true_err = metrics.row_errors(bad[bad_row:bad_row + 1].numpy(), ref)[0]
    assert true_err > 5e-2, true_err
    ok, emax, worst = checks.row_projection_check(Xt, bad, U, G, c)
    assert not ok and worst == bad_row, (emax, worst)
    # a projection of whole 256-row tiles onto one random vector dilutes the same
    # defect below the gate (the reason the row-wise check replaced it)
    w = np.random.default_rng(2).standard_normal(256)
    yt = w @ bad.numpy()[:256]
    exp = oracle.lora_linear_drows(w @ X[:256].astype(np.float64), W0, A, B)
    assert metrics.gemm_ok(yt[None, :], exp)[0]


def test_row_projection_catches_nan_and_zero_rows():
    M, K, N = 64, 1024, 1024
    W0, A, B = _layer(K, N, seed=0)
    X = inputs.activations(0, M, K).float().numpy()
    U, G, c = checks.projection(N, K, W0, A, B, k=16, seed=3)
    Y = _simulated_gpu_output(X, W0, A, B)
    for planted in (np.nan, 0.0):
        Yb = Y.copy()
        Yb[9] = planted
        ok, emax, worst = checks.row_projection_check(torch.from_numpy(X), torch.from_numpy(Yb),
                                                      U, G, c)
        assert not ok and worst == 9
