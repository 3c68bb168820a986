"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases compare every output element; full-size cases (768P, 2K, the
whole 4K grid chunk by chunk, the 2K three-step stand-in) compare sampled rows
exactly and, for the linear layers without SwiGLU, EVERY row through 16 random
column projections (Freivalds' identity on the output columns, tests/checks.py:
Y_i·U against X_i·G + c with the oracle's adjoint G = W0ᵀU + s·Aᵀ(BᵀU)), so a
defect in a single row is not diluted by the others.  Gates: bf16 GEMM outputs
max-over-rows rel-L2 and rel-max <= 2e-2 (the projected statistic estimates the
row's rel-L2); fp32 sampler per-token rel-L2 <= 1e-5; merge bit-exact.
"""
import math

import numpy as np
import pytest
import torch

import checks
import few_step_diffusion_amd as fsd
import oracle
from oracle import metrics
from few_step_diffusion_amd import inputs, schedules
from few_step_diffusion_amd.refine import StandinRefiner

pytestmark = pytest.mark.gpu

TOL = metrics.GEMM_TOL


def say(msg):
    print(f"[case] {msg}", flush=True)


def f32(t):
    return t.detach().float().cpu().numpy()


def bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def merged(wid, K, N, dev, layer=0, ranks=inputs.RANKS, scales=None):
    """Merged adapters on the device (HIP merge) and their oracle float values."""
    A_l, B_l = inputs.adapters(wid, K, N, layer=layer, ranks=ranks)
    A, B = fsd.lora_merge([a.to(dev) for a in A_l], [b.to(dev) for b in B_l], scales)
    Ab, Bb = oracle.merge_bf16([a.numpy() for a in A_l], [b.numpy() for b in B_l], scales)
    return A, B, oracle.bf16_value(Ab).reshape(Ab.shape), oracle.bf16_value(Bb).reshape(Bb.shape)


def assert_gemm(Y, ref, what):
    ok, err = metrics.gemm_ok(Y, ref)
    say(f"{what}: rel_l2 {err[0]:.3e} rel_max {err[1]:.3e}")
    assert ok, (what, err)


def check_all_rows(X, Y, W0f, Af, Bf, bias=None, scale=1.0, residual=None, seed=0, what=""):
    """Every row of Y = X·W0ᵀ + s(X·Aᵀ)·Bᵀ + bias (+ residual) through 16 column projections."""
    N, K = W0f.shape
    U, G, c = checks.projection(N, K, W0f, Af, Bf, scale=scale, bias=bias, k=16, seed=seed)
    ok, emax, worst = checks.row_projection_check(X, Y, U, G, c, residual=residual)
    say(f"{what}: every row through 16 projections, max {emax:.3e} (row {worst})")
    assert ok, (what, emax, worst)


# ----------------------------------------------------------------- merge
def test_merge_bit_exact(gpu):
    say("merge K=N=1024 ranks 384|128|64, scales 1, 0.7, 1.3")
    for scales in (None, [1.0, 0.7, 1.3]):
        A_l, B_l = inputs.adapters(0, 1024, 1024)
        A, B = fsd.lora_merge([a.to(gpu) for a in A_l], [b.to(gpu) for b in B_l], scales)
        Ab, Bb = oracle.merge_bf16([a.numpy() for a in A_l], [b.numpy() for b in B_l], scales)
        torch.cuda.synchronize()
        assert np.array_equal(bits(A), Ab)
        assert np.array_equal(bits(B), Bb)


# ------------------------------------------------------------ small GEMMs
def test_lora_linear_tiny_all_rows(gpu):
    wl = inputs.WORKLOADS[0]
    _, K, N, _ = wl.linears[0]
    M = wl.tokens
    say(f"tiny workload M={M} K={K} N={N} r=576 bias")
    X = inputs.activations(0, M, K)
    W0 = inputs.base_weight(0, K, N)
    bias = inputs.bias(0, N)
    A, B, Af, Bf = merged(0, K, N, gpu)
    Y = fsd.lora_linear(X.to(gpu), W0.to(gpu), A, B, bias=bias.to(gpu))
    ref = oracle.lora_linear_rows(f32(X), f32(W0), Af, Bf, bias=bias.numpy())
    assert_gemm(f32(Y), ref, "tiny")


@pytest.mark.parametrize("M", [1, 17, 255, 256, 257, 300, 513])
@pytest.mark.parametrize("r,scale", [(64, 1.0), (0, 1.0), (576, 0.5)])
def test_lora_linear_tails(gpu, M, r, scale):
    K, N = 256, 320
    say(f"tails M={M} K={K} N={N} r={r} scale={scale}")
    X = inputs.normal((M, K), 1.0, 11 + M, dtype=torch.bfloat16)
    W0 = inputs.normal((N, K), 0.05, 12, dtype=torch.bfloat16)
    bias = inputs.normal((N,), 0.1, 13)
    if r:
        ranks = (r // 2, r // 4, r // 4)
        A, B, Af, Bf = merged(7, K, N, gpu, ranks=ranks)
    else:
        A = B = Af = Bf = None
    Y = fsd.lora_linear(X.to(gpu), W0.to(gpu), A, B, scale=scale, bias=bias.to(gpu))
    ref = oracle.lora_linear_rows(f32(X), f32(W0), Af, Bf, scale=scale, bias=bias.numpy())
    assert_gemm(f32(Y), ref, f"tails M={M} r={r}")


@pytest.mark.parametrize("M,F", [(300, 320), (257, 128), (1, 64)])
def test_swiglu(gpu, M, F):
    K = 512
    say(f"swiglu M={M} K={K} F={F} r=576 bias")
    X = inputs.normal((M, K), 1.0, 21, dtype=torch.bfloat16)
    W0 = inputs.normal((2 * F, K), 0.05, 22, dtype=torch.bfloat16)
    bias = inputs.normal((2 * F,), 0.1, 23)
    A, B, Af, Bf = merged(8, K, 2 * F, gpu)
    H = fsd.lora_linear(X.to(gpu), W0.to(gpu), A, B, bias=bias.to(gpu), epilogue="swiglu")
    ref = oracle.lora_linear_rows(f32(X), f32(W0), Af, Bf, bias=bias.numpy(), swiglu=True)
    assert H.shape == (M, F)
    assert_gemm(f32(H), ref, f"swiglu M={M} F={F}")


def test_residual_separate_and_in_place(gpu):
    M, K, N = 600, 384, 256
    say(f"residual M={M} K={K} N={N}")
    X = inputs.normal((M, K), 1.0, 31, dtype=torch.bfloat16)
    W0 = inputs.normal((N, K), 0.05, 32, dtype=torch.bfloat16)
    R = inputs.normal((M, N), 1.0, 33, dtype=torch.bfloat16)
    A, B, Af, Bf = merged(9, K, N, gpu, ranks=(32, 16, 16))
    ref = oracle.lora_linear_rows(f32(X), f32(W0), Af, Bf, residual=f32(R))
    Y = fsd.lora_linear(X.to(gpu), W0.to(gpu), A, B, residual=R.to(gpu))
    assert_gemm(f32(Y), ref, "residual separate")
    Rd = R.to(gpu)
    Y2 = fsd.lora_linear(X.to(gpu), W0.to(gpu), A, B, residual=Rd, out=Rd)
    assert Y2.data_ptr() == Rd.data_ptr()
    assert torch.equal(Y2.cpu(), Y.cpu())


@pytest.mark.parametrize("M,K,N,r", [
    (300, 64, 320, 0),      # one K step; a partial second N tile
    (257, 64, 320, 16),     # two K steps
    (513, 128, 256, 64),    # three K steps
    (1, 512, 576, 576),     # one token, 17 K steps, partial third N tile
])
def test_residual_short_k_and_tails(gpu, M, K, N, r):
    """The residual tile rides on the loads of the steps past the end of the
    K loop: short K loops, ragged M and partial N tiles, separate and in place."""
    say(f"residual short K M={M} K={K} N={N} r={r}")
    X = inputs.normal((M, K), 1.0, 51 + M, dtype=torch.bfloat16)
    W0 = inputs.normal((N, K), 0.05, 52, dtype=torch.bfloat16)
    R = inputs.normal((M, N), 1.0, 53, dtype=torch.bfloat16)
    bias = inputs.normal((N,), 0.1, 54)
    if r:
        A, B, Af, Bf = merged(11, K, N, gpu, ranks=(r // 2, r // 4, r // 4))
    else:
        A = B = Af = Bf = None
    ref = oracle.lora_linear_rows(f32(X), f32(W0), Af, Bf, bias=bias.numpy(), residual=f32(R))
    Y = fsd.lora_linear(X.to(gpu), W0.to(gpu), A, B, bias=bias.to(gpu), residual=R.to(gpu))
    assert_gemm(f32(Y), ref, f"residual M={M} K={K} N={N} r={r}")
    Rd = R.to(gpu)
    Y2 = fsd.lora_linear(X.to(gpu), W0.to(gpu), A, B, bias=bias.to(gpu), residual=Rd, out=Rd)
    assert Y2.data_ptr() == Rd.data_ptr()
    assert torch.equal(Y2.cpu(), Y.cpu())


@pytest.mark.parametrize("epi", ["none", "swiglu"])
def test_row_permutation_equivariance(gpu, epi):
    """Permuting the rows of X permutes the rows of Y, bit for bit: a token's
    output does not depend on where its row falls within a 256-row tile (ragged
    M, a partial N tile, bias, LoRA; residual on the plain epilogue)."""
    M, K, N = 700, 320, 320 if epi == "none" else 640
    say(f"row permutation M={M} K={K} N={N} {epi}")
    X = inputs.normal((M, K), 1.0, 61, dtype=torch.bfloat16).to(gpu)
    W0 = inputs.normal((N, K), 0.05, 62, dtype=torch.bfloat16).to(gpu)
    bias = inputs.normal((N,), 0.1, 63).to(gpu)
    A, B, _, _ = merged(12, K, N, gpu, ranks=(32, 16, 16))
    nout = N if epi == "none" else N // 2
    R = inputs.normal((M, nout), 1.0, 64, dtype=torch.bfloat16).to(gpu) if epi == "none" else None
    perm = torch.from_numpy(np.random.default_rng(65).permutation(M)).to(gpu)
    Y = fsd.lora_linear(X, W0, A, B, bias=bias, residual=R, epilogue=epi)
    Yp = fsd.lora_linear(X[perm].contiguous(), W0, A, B, bias=bias,
                         residual=None if R is None else R[perm].contiguous(), epilogue=epi)
    assert torch.equal(Yp, Y[perm])


def test_strided_input_slice(gpu):
    M, D = 300, 256
    say(f"V-slice input M={M} D={D} ld=3D")
    QKV = inputs.normal((M, 3 * D), 1.0, 41, dtype=torch.bfloat16)
    W0 = inputs.normal((D, D), 0.05, 42, dtype=torch.bfloat16)
    A, B, Af, Bf = merged(10, D, D, gpu, ranks=(64, 32, 32))
    Qd = QKV.to(gpu)
    Y = fsd.lora_linear(Qd[:, 2 * D:], W0.to(gpu), A, B)
    ref = oracle.lora_linear_rows(f32(QKV[:, 2 * D:]), f32(W0), Af, Bf)
    assert_gemm(f32(Y), ref, "V slice")


def test_lora_down_alone(gpu):
    M, K = 700, 1024
    say(f"phase A M={M} K={K} r=576 scale=0.75")
    X = inputs.activations(0, M, K)
    A, _, Af, _ = merged(0, K, 64, gpu)
    T = fsd.lora_down(X.to(gpu), A, 0.75)
    ref = 0.75 * oracle.lora_linear_rows(f32(X), Af, None, None)   # X·Aᵀ as a plain linear
    assert_gemm(f32(T), ref, "phase A")


def test_chunked_workspace_is_bitwise_identical(gpu):
    """Every schedule of fsd_lora_linear gives the bits of the unchunked one:
    256-row chunks (one buffer), pipelined pairs of 256- to 1024-row chunks,
    the whole of T; plain, SwiGLU and in-place residual epilogues."""
    M, K, N = 5000 + 37, 512, 512
    X = inputs.normal((M, K), 1.0, 51, dtype=torch.bfloat16).to(gpu)
    W0 = inputs.normal((N, K), 0.05, 52, dtype=torch.bfloat16).to(gpu)
    R0 = inputs.normal((M, N), 1.0, 53, dtype=torch.bfloat16).to(gpu)
    A, B, _, _ = merged(11, K, N, gpu)
    for epi, res in (("none", False), ("swiglu", False), ("none", True)):
        say(f"chunking M={M} epilogue={epi} residual={res}")
        whole_ws = torch.empty(M * 576 * 2, dtype=torch.uint8, device=gpu)
        assert fsd.lora_linear_plan(M, 576, whole_ws.numel())[2] == 0
        Y0 = R0.clone() if res else None
        full = fsd.lora_linear(X, W0, A, B, epilogue=epi, residual=Y0, out=Y0,
                               workspace=whole_ws)
        for rows, sched in ((256, 2), (300, 2), (512, 1), (700, 1), (2048, 1)):
            ws = torch.empty(rows * 576 * 2, dtype=torch.uint8, device=gpu)
            assert fsd.lora_linear_plan(M, 576, ws.numel())[2] == sched
            Yc = R0.clone() if res else None
            part = fsd.lora_linear(X, W0, A, B, epilogue=epi, residual=Yc, out=Yc, workspace=ws)
            assert torch.equal(part, full), (epi, res, rows)


def test_launch_by_launch_equals_the_whole_call(gpu):
    """fsd_lora_linear_launch over every index of the plan is fsd_lora_linear."""
    M, K, N = 3000, 512, 1024
    X = inputs.normal((M, K), 1.0, 54, dtype=torch.bfloat16).to(gpu)
    W0 = inputs.normal((N, K), 0.05, 55, dtype=torch.bfloat16).to(gpu)
    A, B, _, _ = merged(13, K, N, gpu)
    ws = torch.empty(1024 * 576 * 2, dtype=torch.uint8, device=gpu)
    seen = []
    a = fsd.lora_linear(X, W0, A, B, workspace=ws)
    b = fsd.lora_linear(X, W0, A, B, workspace=ws, on_launch=seen.append)
    n, R, sched = fsd.lora_linear_plan(M, 576, ws.numel())
    say(f"launch by launch: {n} launches, chunks of {R}, schedule {sched}")
    assert seen == list(range(n)) and sched == 1 and R == 512
    assert torch.equal(a, b)


def test_chunked_schedule_is_bitwise_identical_at_2k(gpu):
    """The 2K QKV linear through the default 50 MB workspace (pipelined pairs of
    21,760-row chunks) against the whole of T in one 614 MB workspace."""
    wid = 2
    _, K, N, _ = inputs.WORKLOADS[wid].linears[0]
    M = inputs.WORKLOADS[wid].tokens
    X = inputs.activations(wid, M, K, device=gpu)
    W0 = inputs.base_weight(wid, K, N).to(gpu)
    A, B, _, _ = merged(wid, K, N, gpu)
    small = torch.empty(fsd.workspace_bytes(M, 576), dtype=torch.uint8, device=gpu)
    n, R, sched = fsd.lora_linear_plan(M, 576, small.numel())
    say(f"2K QKV: default workspace {small.numel() / 1e6:.1f} MB, {n} launches of "
        f"{R}-row chunks (schedule {sched}) vs the whole of T")
    assert sched == 1 and R == 21760 and small.numel() <= 64e6
    Ya = fsd.lora_linear(X, W0, A, B, workspace=small)
    del small
    whole = torch.empty(M * 576 * 2, dtype=torch.uint8, device=gpu)
    Yb = fsd.lora_linear(X, W0, A, B, workspace=whole)
    torch.cuda.synchronize()
    assert torch.equal(Ya, Yb)
    del X, Ya, Yb, whole
    torch.cuda.empty_cache()


def test_determinism(gpu):
    M, K, N = 4099, 1024, 2048
    say(f"determinism M={M} K={K} N={N}")
    X = inputs.normal((M, K), 1.0, 61, dtype=torch.bfloat16).to(gpu)
    W0 = inputs.normal((N, K), 0.02, 62, dtype=torch.bfloat16).to(gpu)
    A, B, _, _ = merged(12, K, N, gpu)
    a = fsd.lora_linear(X, W0, A, B)
    b = fsd.lora_linear(X, W0, A, B)
    c = fsd.lora_linear(X, W0, A, B, epilogue="swiglu")
    d = fsd.lora_linear(X, W0, A, B, epilogue="swiglu")
    assert torch.equal(a, b) and torch.equal(c, d)


def test_nan_propagates_to_its_row_only(gpu):
    M, K, N = 300, 256, 256
    say("NaN row propagation")
    X = inputs.normal((M, K), 1.0, 71, dtype=torch.bfloat16)
    X[5, 17] = float("nan")
    W0 = inputs.normal((N, K), 0.05, 72, dtype=torch.bfloat16)
    A, B, _, _ = merged(13, K, N, gpu, ranks=(32, 16, 16))
    Y = fsd.lora_linear(X.to(gpu), W0.to(gpu), A, B).cpu()
    assert torch.isnan(Y[5]).all()
    rest = torch.cat([Y[:5], Y[6:]])
    assert torch.isfinite(rest).all()


# ---------------------------------------------------------------- sampler
def _sampler(gpu, x0, eps, in_place=False):
    xd, ed = x0.to(gpu), eps.to(gpu)
    if in_place:
        z = xd.clone()
        fsd.renoise(z, ed, oracle.SIGMAS[0], out=z)
    else:
        z = fsd.renoise(xd, ed, oracle.SIGMAS[0])
    hist = [z.cpu().clone()]
    v = ed - xd           # the exact flow-matching velocity, an input of the Euler step
    for k in range(3):
        fsd.euler_step(z, v, oracle.SIGMAS[k], oracle.SIGMAS[k + 1])
        hist.append(z.cpu().clone())
    return hist


@pytest.mark.parametrize("wid", [0, 1, 2, 3])
def test_sampler_full_latent(gpu, wid):
    wl = inputs.WORKLOADS[wid]
    say(f"sampler {wl.name}: {wl.latent_elems} elements")
    x0, eps = inputs.latent(wid)
    hist = _sampler(gpu, x0, eps, in_place=(wid == 0))
    ref = oracle.sampler_exact_velocity(x0.numpy(), eps.numpy())
    for k in range(4):
        e = metrics.token_error(hist[k].numpy(), ref[k])
        say(f"  sigma={oracle.SIGMAS[k]} token err {e:.2e}")
        assert e <= metrics.SAMPLER_TOL, (k, e)
    # closed form: the last step lands on x0
    assert float((hist[-1] - x0).abs().max()) <= 1e-5


@pytest.mark.parametrize("route", ["up3", "up4", "hf8"])
def test_ic_sampler_routes(gpu, route):
    """The in-context routes on the 768P latent: renoise at the route's start, then
    one Euler step per table target, every step against the oracle; the last step
    lands on x0 (closed form, exact velocity)."""
    sig = schedules.route(route)
    x0, eps = inputs.latent(1)
    say(f"IC route {route}: sigmas {[round(x, 4) for x in sig]}, {x0.numel()} elements")
    xd, ed = x0.to(gpu), eps.to(gpu)
    z = fsd.renoise(xd, ed, sig[0])
    hist = [z.cpu().clone()]
    v = ed - xd
    for k in range(len(sig) - 1):
        fsd.euler_step(z, v, sig[k], sig[k + 1])
        hist.append(z.cpu().clone())
    ref = oracle.sampler_exact_velocity(x0.numpy(), eps.numpy(), oracle.ic_route(route))
    for k in range(len(sig)):
        e = metrics.token_error(hist[k].numpy(), ref[k])
        assert e <= metrics.SAMPLER_TOL, (route, k, e)
    assert float((hist[-1] - x0).abs().max()) <= 1e-5


def test_reference_row_renoise(gpu):
    """The reference row of the IC routes: 99.9% draft + 0.1% noise."""
    x0, eps = inputs.latent(1)
    z = fsd.renoise(x0.to(gpu), eps.to(gpu), schedules.REFERENCE_ROW_SIGMA)
    ref = oracle.renoise(x0.numpy(), eps.numpy(), oracle.REFERENCE_ROW_SIGMA)
    assert metrics.token_error(z.cpu().numpy(), ref) <= metrics.SAMPLER_TOL


@pytest.mark.parametrize("n", [0, 1, 3, 4, 5, 7, 1023, 4099])
def test_sampler_ragged_lengths(gpu, n):
    say(f"sampler flat n={n}")
    u = inputs.normal((n,), 1.0, 81)
    e = inputs.normal((n,), 1.0, 82)
    z = fsd.renoise(u.to(gpu), e.to(gpu), 0.909)
    v = (e - u).to(gpu)
    fsd.euler_step(z, v, 0.909, 0.857)
    ref = oracle.euler_step(oracle.renoise(u.numpy(), e.numpy(), 0.909),
                            e.numpy().astype(np.float64) - u.numpy(), 0.909, 0.857)
    got = z.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1e-6 * np.maximum(1.0, np.abs(ref)))


def test_sampler_nan_propagates(gpu):
    u = torch.zeros(64)
    u[10] = float("nan")
    z = fsd.renoise(u.to(gpu), torch.ones(64, device=gpu), 0.909).cpu()
    assert math.isnan(float(z[10])) and torch.isfinite(torch.cat([z[:10], z[11:]])).all()


# ---------------------------------------------------------- embed / head
def test_embed_and_head(gpu):
    M, C, D = 1000, 24, 3072
    say(f"embed/head M={M} C={C} D={D}")
    z = inputs.normal((M, C), 1.0, 91)
    E, P = inputs.standin_projections(4, C, D)
    X = fsd.token_embed(z.to(gpu), E.to(gpu))
    assert_gemm(f32(X), oracle.embed_rows(z.numpy(), f32(E)), "embed")
    H = inputs.normal((M, D), 1.0, 92, dtype=torch.bfloat16)
    v = fsd.token_head(H.to(gpu), P.to(gpu))
    assert_gemm(v.cpu().numpy(), oracle.head_rows(f32(H), f32(P)), "head")


@pytest.mark.parametrize("M,C,D", [(1, 1, 64), (65, 7, 96), (129, 32, 192), (300, 24, 1000),
                                   (64, 8, 576)])
def test_embed_shapes(gpu, M, C, D):
    """Tails in tokens (past 128 per wave), in columns (odd 32-column tile
    counts, D not a multiple of 32 or of the 512-column wave range), and the
    scalar E path (C not a multiple of 8)."""
    say(f"embed M={M} C={C} D={D}")
    z = inputs.normal((M, C), 1.0, 93)
    E, _ = inputs.standin_projections(4, C, D)
    X = fsd.token_embed(z.to(gpu), E.to(gpu))
    assert_gemm(f32(X), oracle.embed_rows(z.numpy(), f32(E)), "embed")


@pytest.mark.parametrize("M,C,D", [(1, 1, 64), (63, 7, 128), (65, 32, 192), (1000, 24, 640)])
def test_head_shapes(gpu, M, C, D):
    """Row tails around the 64-row block, every C up to 32, short K loops."""
    say(f"head M={M} C={C} D={D}")
    _, P = inputs.standin_projections(4, C, D)
    H = inputs.normal((M, D), 1.0, 94, dtype=torch.bfloat16)
    v = fsd.token_head(H.to(gpu), P.to(gpu))
    assert_gemm(v.cpu().numpy(), oracle.head_rows(f32(H), f32(P)), "head")


def test_head_euler_fused(gpu):
    """z += (σ'−σ)·H·Pᵀ in one kernel: against the oracle's head then Euler step,
    and bit for bit against the unfused route (same fp32 sums, same fma)."""
    M, C, D = 1000, 24, 3072
    say(f"head+Euler M={M} C={C} D={D}")
    H = inputs.normal((M, D), 1.0, 95, dtype=torch.bfloat16)
    _, P = inputs.standin_projections(4, C, D)
    z0 = inputs.normal((M, C), 1.0, 96)
    Hd, Pd = H.to(gpu), P.to(gpu)
    z = z0.to(gpu).clone()
    fsd.token_head_euler(Hd, Pd, z, 0.857, 0.667)
    z_ref = oracle.euler_step(z0.numpy(), oracle.head_rows(f32(H), f32(P)), 0.857, 0.667)
    e = metrics.token_error(z.cpu().numpy(), z_ref)
    say(f"  token err {e:.3e}")
    assert e <= metrics.SAMPLER_TOL
    z2 = z0.to(gpu).clone()
    fsd.euler_step(z2, fsd.token_head(Hd, Pd), 0.857, 0.667)
    assert torch.equal(z, z2)


def test_refine_fused_and_step_graphs(gpu):
    """The refine with the head+Euler kernel equals the unfused refine bit for bit;
    one HIP graph per sampler step, replayed with eager work and synchronisations
    between replays, reproduces it on every replay."""
    M = 4096 + 37
    say(f"stand-in refine M={M}: fused and graph replays")
    model = StandinRefiner(M, device=gpu)
    u, eps = inputs.latent(4, tokens=M)
    u, eps = u.to(gpu), eps.to(gpu)
    z_ref = model.refine(u, eps).clone()
    z_fused = model.refine(u, eps, fused=True).clone()
    assert torch.equal(z_ref, z_fused)
    graphs = model.capture_steps(fused=True)
    for rep in range(3):
        noise = torch.randn(1 << 20, device=gpu)
        _ = (noise * 2.0).sum().item()                 # eager work + a synchronisation
        model.z.fill_(float("nan"))
        z_g = model.refine_graphs(graphs, u, eps).clone()
        torch.cuda.synchronize()
        say(f"  replay {rep}: equal {torch.equal(z_g, z_ref)}")
        assert torch.equal(z_g, z_ref), rep
    del model, graphs
    torch.cuda.empty_cache()


# ------------------------------------------------------- full-size shapes
def _full_linear(gpu, wid, label, K, N, layer=0, M=None, rows=384):
    M = inputs.WORKLOADS[wid].tokens if M is None else M
    say(f"{inputs.WORKLOADS[wid].name}: {label} M={M} K={K} N={N} r=576")
    X = inputs.activations(wid, M, K, device=gpu, layer=layer)
    W0 = inputs.base_weight(wid, K, N, layer=layer)
    A, B, Af, Bf = merged(wid, K, N, gpu, layer=layer)
    W0d = W0.to(gpu)
    Y = fsd.lora_linear(X, W0d, A, B)
    torch.cuda.synchronize()
    sel = inputs.sample_rows(M, rows, seed=wid * 10 + layer)
    seli = torch.from_numpy(sel).to(gpu)
    ref = oracle.lora_linear_rows(f32(X[seli]), f32(W0), Af, Bf)
    assert_gemm(f32(Y[seli]), ref, f"{label} sampled rows")
    check_all_rows(X, Y, f32(W0), Af, Bf, seed=wid, what=label)
    del X, Y
    torch.cuda.empty_cache()


def test_full_768p(gpu):
    _, K, N, _ = inputs.WORKLOADS[1].linears[0]
    _full_linear(gpu, 1, "768P linear", K, N)


def test_full_2k_qkv_and_o(gpu):
    for layer, (label, K, N, _) in enumerate(inputs.WORKLOADS[2].linears):
        _full_linear(gpu, 2, f"2K {label}", K, N, layer=layer)


def test_full_2k_o_strided_in_place(gpu):
    """The O linear exactly as the step runs it: input the V slice of a
    [M, 9216] QKV buffer (row stride 9216), residual added in place into h."""
    wid = 2
    _, K, N, _ = inputs.WORKLOADS[wid].linears[1]
    M = inputs.WORKLOADS[wid].tokens
    say(f"2K O linear M={M}: V slice input (ld {3 * K}), in-place residual")
    qkv = inputs.activations(wid, M, 3 * K, device=gpu, layer=5)
    V = qkv[:, 2 * K:3 * K]
    h = inputs.normal((M, N), 1.0, seed=2077, device=gpu, dtype=torch.bfloat16)
    h0 = h.clone()
    W0 = inputs.base_weight(wid, K, N, layer=1)
    A, B, Af, Bf = merged(wid, K, N, gpu, layer=1)
    fsd.lora_linear(V, W0.to(gpu), A, B, residual=h, out=h)
    torch.cuda.synchronize()
    sel = torch.from_numpy(inputs.sample_rows(M, 256, seed=21)).to(gpu)
    ref = oracle.lora_linear_rows(f32(V[sel]), f32(W0), Af, Bf) + f32(h0[sel])
    assert_gemm(f32(h[sel]), ref, "2K O (V slice, in place) sampled rows")
    check_all_rows(V, h, f32(W0), Af, Bf, residual=h0, seed=22, what="2K O (V slice, in place)")
    del qkv, V, h, h0
    torch.cuda.empty_cache()


def test_full_4k_whole_grid(gpu):
    """The whole 4K grid (1,198,800 tokens) as its four 299,700-token chunks run
    it, one after another through shared buffers and one workspace: gate/up with
    SwiGLU (K = 3072 -> 2 x 8192), then down (8192 -> 3072) with the gate/up
    input added as the residual.  Per chunk: 40 sampled rows of H and of Y
    against the oracle's chain (its own H feeding its down), and every row of Y
    through 16 column projections given the GPU's H."""
    wl = inputs.WORKLOADS[3]
    Mc = wl.tokens // wl.chunks
    (_, K1, N1, _), (_, K2, N2, _) = wl.linears
    say(f"{wl.name}: {wl.chunks} chunks of {Mc}, gate/up {K1}->{N1} SwiGLU, "
        f"down {K2}->{N2} + residual")
    Xall = inputs.activations(3, wl.tokens, K1, device=gpu)
    W1 = inputs.base_weight(3, K1, N1, layer=1)
    W2 = inputs.base_weight(3, K2, N2, layer=2)
    W1d, W2d = W1.to(gpu), W2.to(gpu)
    W1f, W2f = f32(W1), f32(W2)
    A1, B1, A1f, B1f = merged(3, K1, N1, gpu, layer=1)
    A2, B2, A2f, B2f = merged(3, K2, N2, gpu, layer=2)
    H = torch.empty((Mc, N1 // 2), dtype=torch.bfloat16, device=gpu)
    Y = torch.empty((wl.tokens, N2), dtype=torch.bfloat16, device=gpu)
    ws = torch.empty(fsd.workspace_bytes(Mc, A1.shape[0]), dtype=torch.uint8, device=gpu)
    for c in range(wl.chunks):
        rows = slice(c * Mc, (c + 1) * Mc)
        X, Yc = Xall[rows], Y[rows]
        say(f"  chunk {c}: rows {c * Mc}-{(c + 1) * Mc - 1}")
        fsd.lora_linear(X, W1d, A1, B1, epilogue="swiglu", out=H, workspace=ws)
        fsd.lora_linear(H, W2d, A2, B2, residual=X, out=Yc, workspace=ws)
        torch.cuda.synchronize()
        sel = inputs.sample_rows(Mc, 40, seed=3 + c)
        seli = torch.from_numpy(sel).to(gpu)
        Href = oracle.lora_linear_rows(f32(X[seli]), W1f, A1f, B1f, swiglu=True)
        assert_gemm(f32(H[seli]), Href, f"4K chunk {c} gate/up SwiGLU sampled rows")
        # the chain from X in fp64: the oracle's H (not the GPU's) feeds its down projection
        Yref = oracle.lora_linear_drows(Href, W2f, A2f, B2f) + f32(X[seli])
        assert_gemm(f32(Yc[seli]), Yref, f"4K chunk {c} down (chained, residual) sampled rows")
        check_all_rows(H, Yc, W2f, A2f, B2f, residual=X, seed=31 + c,
                       what=f"4K chunk {c} down")
    del Xall, H, Y, ws
    torch.cuda.empty_cache()


def test_full_2k_standin_three_steps(gpu):
    wl = inputs.WORKLOADS[4]
    M = wl.tokens
    say(f"{wl.name}: M={M}, 3 steps")
    ref_model = StandinRefiner(M, device=gpu)
    u, eps = inputs.latent(4)
    z = ref_model.refine(u.to(gpu), eps.to(gpu)).cpu().numpy()
    assert np.all(np.isfinite(z))
    sel = inputs.sample_rows(M, 24, seed=4)
    layers = []
    for L in inputs.standin_layers(4):
        Ab, Bb = oracle.merge_bf16([a.numpy() for a in L["A_list"]],
                                   [b.numpy() for b in L["B_list"]])
        layers.append({"W0": f32(L["W0"]), "A": oracle.bf16_value(Ab).reshape(Ab.shape),
                       "B": oracle.bf16_value(Bb).reshape(Bb.shape)})
    E, P = inputs.standin_projections(4)
    zh, vh = oracle.standin_refine(u.numpy()[sel], eps.numpy()[sel], f32(E), f32(P), layers)
    e = metrics.token_error(z[sel], zh[-1])
    say(f"  final latent token err {e:.3e}")
    assert e <= TOL
    # the velocity of the last step, against the oracle's (bf16-path tolerance)
    assert_gemm(ref_model.v.cpu().numpy()[sel], vh[-1], "stand-in velocity, step 3")
    del ref_model
    torch.cuda.empty_cache()
