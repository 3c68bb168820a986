"""Invariants that pin the oracle to the pages and to mathematics.

  merge        B·A equals the sum of the separate adapter deltas; order matters;
               the bf16 storage form equals torch's RNE cast bit for bit.
  sampler      Euler with the exact flow-matching velocity lands on every
               z_sigma of the schedule and on x0 at sigma = 0 (closed form);
               renoise reduces to u at sigma 0 and to eps at sigma 1.
  reductions   s = 0 / r = 0 give the plain GEMM; X = I reveals W0 + s·B·A;
               X = 0 gives the bias; permuting rows permutes outputs.
  SwiGLU       textbook values of silu; gate/up order.
  stand-in     with sublayers zeroed it collapses to closed forms computed
               through merged weights (a different algebraic route).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from few_step_diffusion_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, *vals = line.split()
                out[key] = [float(v) for v in vals]
    return out


# ------------------------------------------------------------------ merge
def _small_adapters(seed, K=48, N=40, ranks=(12, 6, 3)):
    g = np.random.Generator(np.random.PCG64(seed))
    A = [(g.standard_normal((r, K)) / np.sqrt(K)).astype(np.float32) for r in ranks]
    B = [(g.standard_normal((N, r)) * 0.01).astype(np.float32) for r in ranks]
    return A, B


def test_merge_equals_sum_of_adapters():
    A_l, B_l = _small_adapters(1)
    scales = [1.0, 0.5, 2.0]
    A, B = oracle.merge(A_l, B_l, scales)
    ref = sum(s * (b.astype(np.float64) @ a.astype(np.float64))
              for s, a, b in zip(scales, A_l, B_l))
    assert np.linalg.norm(B @ A - ref) / np.linalg.norm(ref) <= 1e-13


def test_merge_at_page_ranks_fp64_and_fp32():
    g = _golden("merge.txt")
    ranks = tuple(int(r) for r in g["ranks"])
    assert sum(ranks) == int(g["merged_rank"][0])
    K = N = 1024
    A_l, B_l = inputs.adapters(0, K, N, ranks=ranks)
    A_l = [a.numpy() for a in A_l]
    B_l = [b.numpy() for b in B_l]
    A, B = oracle.merge(A_l, B_l)
    assert A.shape == (576, K) and B.shape == (N, 576)
    ref = sum(b.astype(np.float64) @ a.astype(np.float64) for a, b in zip(A_l, B_l))
    assert np.linalg.norm(B @ A - ref) / np.linalg.norm(ref) <= 1e-13
    # In fp32 the merged delta differs from the separate ones only by rounding,
    # the level of the pages' merge check (their weights are not available, so
    # only the order of magnitude is comparable): far below the O(1) error of a
    # wrong merge.
    m32 = torch.from_numpy(B.astype(np.float32)) @ torch.from_numpy(A.astype(np.float32))
    s32 = sum(torch.from_numpy(b) @ torch.from_numpy(a) for a, b in zip(A_l, B_l))
    rel32 = float((m32 - s32).norm() / s32.norm())
    page = g["fp32_relative_error"][0]
    assert rel32 < 1e-6 and page < 1e-6


def test_merge_order_is_pinned():
    A_l, B_l = _small_adapters(2)
    A, B = oracle.merge(A_l, B_l)
    ref = sum(b.astype(np.float64) @ a.astype(np.float64) for a, b in zip(A_l, B_l))
    # the same permutation of adapters on both factors is still a valid merge...
    Ap, Bp = oracle.merge([A_l[0], A_l[2], A_l[1]], [B_l[0], B_l[2], B_l[1]])
    assert np.linalg.norm(Bp @ Ap - ref) / np.linalg.norm(ref) <= 1e-13
    # ...permuting the row blocks of A alone is not
    A_sw = np.concatenate([A[:12], A[18:21], A[12:18]])
    assert np.linalg.norm(B @ A_sw - ref) / np.linalg.norm(ref) > 0.5


def test_merge_bf16_matches_torch_cast():
    A_l, B_l = _small_adapters(3)
    scales = [1.0, 0.3, 1.7]
    Ab, Bb = oracle.merge_bf16(A_l, B_l, scales)
    A_t = torch.cat([torch.from_numpy(a) for a in A_l]).to(torch.bfloat16)
    B_t = torch.cat([torch.from_numpy(b) * s for s, b in zip(scales, B_l)], dim=1).to(torch.bfloat16)
    assert np.array_equal(Ab, A_t.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(Bb, B_t.view(torch.int16).numpy().view(np.uint16))


def test_bf16_rounding_matches_torch_including_ties():
    g = np.random.Generator(np.random.PCG64(5))
    x = g.standard_normal(4000).astype(np.float32) * np.float32(3.0)
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    edge = np.array([0.0, -0.0, 1e-40, -1e-40, 3.3895e38, np.inf, -np.inf, 1.0, 65504.0],
                    dtype=np.float32)
    vals = np.concatenate([x, ties, -ties, edge])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits(vals), ref)


# ------------------------------------------------------------------ sampler
def test_schedule_matches_pages():
    g = _golden("schedule.txt")
    assert tuple(oracle.SIGMAS) == tuple(g["schedule"])
    assert oracle.SIGMAS[0] == g["sigma0"][0]
    assert len(oracle.SIGMAS) - 1 == int(g["steps"][0])


def test_euler_with_exact_velocity_follows_closed_form():
    x0, eps = inputs.latent(0)
    x0, eps = x0.numpy(), eps.numpy()
    z = oracle.sampler_exact_velocity(x0, eps)
    X, E = x0.astype(np.float64), eps.astype(np.float64)
    for k, s in enumerate(oracle.SIGMAS):
        closed = (1.0 - s) * X + s * E
        assert np.abs(z[k] - closed).max() <= 1e-15 * max(1.0, np.abs(closed).max()) * 8, k
    # the last step lands on x0
    assert np.abs(z[-1] - X).max() <= 1e-14


def test_euler_sign_matters():
    x0, eps = inputs.latent(0, tokens=50)
    x0, eps = x0.numpy().astype(np.float64), eps.numpy().astype(np.float64)
    z = (1 - 0.909) * x0 + 0.909 * eps
    v = eps - x0
    good = oracle.euler_step(z, v, 0.909, 0.857)
    assert np.allclose(good, (1 - 0.857) * x0 + 0.857 * eps, atol=1e-14)
    bad = oracle.euler_step(z, -v, 0.909, 0.857)
    assert not np.allclose(bad, (1 - 0.857) * x0 + 0.857 * eps, atol=1e-3)


def test_renoise_special_cases():
    u, e = inputs.latent(0, tokens=64)
    assert np.array_equal(oracle.renoise(u, e, 0.0), u.numpy().astype(np.float64))
    assert np.array_equal(oracle.renoise(u, e, 1.0), e.numpy().astype(np.float64))
    half = oracle.renoise(u, e, 0.5)
    assert np.allclose(half, 0.5 * (u.numpy() + e.numpy()), atol=1e-7)


# ------------------------------------------------------------ reductions
def _layer(seed, K, N, r):
    g = np.random.Generator(np.random.PCG64(seed))
    X = g.standard_normal((17, K)).astype(np.float32)
    W0 = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = (g.standard_normal((r, K)) / np.sqrt(K)).astype(np.float32)
    B = (g.standard_normal((N, r)) * 0.01).astype(np.float32)
    bias = (g.standard_normal(N) * 0.02).astype(np.float32)
    return X, W0, A, B, bias


def test_scale_zero_and_rank_zero_give_plain_gemm():
    X, W0, A, B, _ = _layer(10, 32, 24, 8)
    plain = X.astype(np.float64) @ W0.T.astype(np.float64)
    assert np.allclose(oracle.lora_linear_rows(X, W0, A, B, scale=0.0), plain, rtol=0, atol=1e-13)
    assert np.allclose(oracle.lora_linear_rows(X, W0, None, None), plain, rtol=0, atol=1e-13)


def test_identity_input_reveals_merged_weight():
    K, N, r, s = 24, 16, 6, 0.75
    _, W0, A, B, _ = _layer(11, K, N, r)
    Y = oracle.lora_linear_rows(np.eye(K, dtype=np.float32), W0, A, B, scale=s)
    merged = W0.astype(np.float64) + s * B.astype(np.float64) @ A.astype(np.float64)
    assert np.allclose(Y, merged.T, rtol=0, atol=1e-15)


def test_zero_input_gives_bias():
    X, W0, A, B, bias = _layer(12, 16, 8, 4)
    Y = oracle.lora_linear_rows(np.zeros_like(X), W0, A, B, bias=bias)
    assert np.array_equal(Y, np.broadcast_to(bias.astype(np.float64), Y.shape))


def test_row_permutation_equivariance():
    X, W0, A, B, bias = _layer(13, 40, 24, 8)
    perm = np.random.Generator(np.random.PCG64(1)).permutation(X.shape[0])
    Y = oracle.lora_linear_rows(X, W0, A, B, bias=bias)
    Yp = oracle.lora_linear_rows(X[perm], W0, A, B, bias=bias)
    assert np.array_equal(Yp, Y[perm])


def test_residual_is_added():
    X, W0, A, B, bias = _layer(14, 16, 8, 4)
    res = np.random.Generator(np.random.PCG64(2)).standard_normal((17, 8)).astype(np.float32)
    Y = oracle.lora_linear_rows(X, W0, A, B, bias=bias)
    Yr = oracle.lora_linear_rows(X, W0, A, B, bias=bias, residual=res)
    assert np.allclose(Yr - Y, res.astype(np.float64), atol=1e-15)


# ------------------------------------------------------------------ SwiGLU
def _swiglu_of(g_vals, u_vals):
    """Drive the SwiGLU epilogue through X = I: row k of Y is column k of W0ᵀ."""
    F = len(g_vals)
    W0 = np.zeros((2 * F, 1), np.float32)
    W0[:F, 0] = g_vals
    W0[F:, 0] = u_vals
    return oracle.lora_linear_rows(np.ones((1, 1), np.float32), W0, None, None, swiglu=True)[0]


def test_swiglu_textbook_values():
    h = _swiglu_of([0.0, 1.0, 40.0, -40.0, 1.0, -1.0], [5.0, 1.0, 0.5, 3.0, -2.0, 1.0])
    assert h[0] == 0.0
    assert abs(h[1] - 1.0 / (1.0 + math.exp(-1.0))) <= 1e-16       # silu(1) = sigmoid(1)
    assert abs(h[1] - 0.7310585786300049) <= 1e-16
    assert abs(h[2] - 40.0 * 0.5) <= 1e-12                         # silu(g) -> g
    assert abs(h[3]) <= 40.0 * 3.0 * math.exp(-40.0) * 1.01        # silu(g) -> 0
    assert abs(h[4] - (-2.0) * 0.7310585786300049) <= 1e-15         # linear in u
    assert abs(h[5] - (-1.0 / (1.0 + math.e))) <= 1e-16            # silu(-1) = -sigmoid(-1)


def test_swiglu_gate_up_order():
    h = _swiglu_of([2.0], [-3.0])
    swapped = _swiglu_of([-3.0], [2.0])
    assert abs(h[0] - 2.0 / (1.0 + math.exp(-2.0)) * -3.0) <= 1e-15
    assert abs(h[0] - swapped[0]) > 1.0


# ---------------------------------------------------------------- stand-in
def _tiny_standin(seed, C=4, D=16, F=24, ranks=(4, 2, 2)):
    g = np.random.Generator(np.random.PCG64(seed))
    E = (g.standard_normal((D, C)) / np.sqrt(C)).astype(np.float32)
    P = (g.standard_normal((C, D)) / np.sqrt(D)).astype(np.float32)
    layers = []
    for K, N in [(D, 3 * D), (D, D), (D, 2 * F), (F, D)]:
        A = [(g.standard_normal((r, K)) / np.sqrt(K)).astype(np.float32) for r in ranks]
        B = [(g.standard_normal((N, r)) * 0.1).astype(np.float32) for r in ranks]
        Am, Bm = oracle.merge(A, B)
        layers.append({"W0": (g.standard_normal((N, K)) * 0.2).astype(np.float32),
                       "A": Am.astype(np.float32), "B": Bm.astype(np.float32), "scale": 1.0})
    x0 = g.standard_normal((9, C)).astype(np.float32)
    eps = g.standard_normal((9, C)).astype(np.float32)
    return E, P, layers, x0, eps


def _merged(L):
    return L["W0"].astype(np.float64) + L["scale"] * L["B"].astype(np.float64) @ L["A"].astype(np.float64)


def _zero(L):
    return dict(L, W0=np.zeros_like(L["W0"]), B=np.zeros_like(L["B"]))


def test_standin_with_zero_sublayers_is_embed_then_head():
    E, P, layers, x0, eps = _tiny_standin(20)
    layers = [layers[0], _zero(layers[1]), layers[2], _zero(layers[3])]
    z = oracle.renoise(x0, eps, 0.909)
    v = oracle.standin_velocity(z, E, P, layers)
    ref = z @ (P.astype(np.float64) @ E.astype(np.float64)).T
    assert np.allclose(v, ref, rtol=0, atol=1e-13)


def test_standin_attention_slice_and_residual():
    E, P, layers, x0, eps = _tiny_standin(21)
    D = E.shape[0]
    layers = [layers[0], layers[1], layers[2], _zero(layers[3])]
    z = oracle.renoise(x0, eps, 0.909)
    v = oracle.standin_velocity(z, E, P, layers)
    x = z @ E.astype(np.float64).T
    Wv = _merged(layers[0])[2 * D:3 * D]          # the V rows of the QKV projection
    h = x + (x @ Wv.T) @ _merged(layers[1]).T
    assert np.allclose(v, h @ P.astype(np.float64).T, rtol=0, atol=1e-12)


def test_standin_mlp_path():
    E, P, layers, x0, eps = _tiny_standin(22)
    F = layers[3]["W0"].shape[1]
    layers = [layers[0], _zero(layers[1]), layers[2], layers[3]]
    z = oracle.renoise(x0, eps, 0.909)
    v = oracle.standin_velocity(z, E, P, layers)
    x = z @ E.astype(np.float64).T
    gu = x @ _merged(layers[2]).T
    g, u = gu[:, :F], gu[:, F:]
    h = x + (g / (1.0 + np.exp(-g)) * u) @ _merged(layers[3]).T
    assert np.allclose(v, h @ P.astype(np.float64).T, rtol=0, atol=1e-12)


def test_standin_refine_runs_the_schedule():
    E, P, layers, x0, eps = _tiny_standin(23)
    z, v = oracle.standin_refine(x0, eps, E, P, layers)
    assert np.array_equal(z[0], oracle.renoise(x0, eps, 0.909))
    for k in range(3):
        vk = oracle.standin_velocity(z[k], E, P, layers)
        assert np.array_equal(v[k], vk)
        step = oracle.euler_step(z[k], vk, oracle.SIGMAS[k], oracle.SIGMAS[k + 1])
        assert np.array_equal(z[k + 1], step)
    # tokens are independent: a subset gives the same rows
    zs, _ = oracle.standin_refine(x0[3:5], eps[3:5], E, P, layers)
    assert np.array_equal(zs, z[:, 3:5])


def test_latent_grids_match_pages():
    g = _golden("latent_grids.txt")
    f, c, h, w = (int(v) for v in g["target_2k"])
    wl = inputs.WORKLOADS[2]
    assert (wl.frames, inputs.LATENT_C, wl.height, wl.width) == (f, c, h, w)
    fd, cd, hd, wd = (int(v) for v in g["draft_2k"])
    assert (fd, cd) == (f, c) and h / hd == 2.5 and w / wd == 2.5
    for key, wid in (("pixels_768p", 1), ("pixels_2k", 2), ("pixels_4k", 3)):
        px_w, px_h = (int(v) for v in g[key])
        wl = inputs.WORKLOADS[wid]
        assert (wl.width, wl.height) == (px_w // 16, px_h // 16)
