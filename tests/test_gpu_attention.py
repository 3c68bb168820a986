"""GPU parity of dense attention (fsd_attention) against the fp64 oracle
(oracle/attention.py).  Q, K and V are the three slices of one QKV buffer, as a
QKV projection writes them.  Gate: per query row, rel-L2 and rel-max of O <= 2e-2
(the bf16 GEMM gate: O is a bf16 product of bf16 inputs with fp32 sums)."""
import numpy as np
import pytest
import torch

import few_step_diffusion_amd as fsd
from oracle import attention, metrics

pytestmark = pytest.mark.gpu

D = 128


def say(msg):
    print(f"[case] {msg}", flush=True)


def qkv_buffer(S, H, seed, dev, peak=1.0):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    qkv = torch.randn((S, 3 * H * D), generator=g, device=dev)
    qkv[:, :2 * H * D] *= peak                     # sharper softmax when peak > 1
    return qkv.to(torch.bfloat16)


def check(qkv, H, rows, what, scale=None):
    HD = H * D
    Q, K, V = qkv[:, :HD], qkv[:, HD:2 * HD], qkv[:, 2 * HD:]
    O = fsd.attention(Q, K, V, H, scale=scale)
    torch.cuda.synchronize()
    got = O[torch.from_numpy(rows).to(qkv.device)].float().cpu().numpy()
    ref = np.empty((len(rows), HD))
    for h in range(H):                             # one head at a time on the host
        cols = slice(h * D, (h + 1) * D)
        ref[:, cols] = attention.attention_rows(
            Q[:, cols].float().cpu().numpy(), K[:, cols].float().cpu().numpy(),
            V[:, cols].float().cpu().numpy(), heads=1, rows=rows, scale=scale)
    ok, err = metrics.gemm_ok(got, ref)
    say(f"{what}: rel_l2 {err[0]:.3e} rel_max {err[1]:.3e}")
    assert ok, (what, err)
    return O


@pytest.mark.parametrize("S,H,peak", [(1, 1, 1.0), (37, 2, 1.0), (300, 3, 1.0), (1200, 4, 1.0),
                                      (4133, 2, 1.0), (700, 1, 3.0)])
def test_attention_all_rows(gpu, S, H, peak):
    """Tails in queries (256 per workgroup) and keys (64 per block), one key and one
    query, several heads, and a sharp softmax (logits scaled 9x) that moves the
    running maximum often."""
    say(f"attention S={S} H={H} peak={peak}")
    qkv = qkv_buffer(S, H, 1000 + S + H, gpu, peak)
    check(qkv, H, np.arange(S), f"attention S={S} H={H}")


def test_attention_custom_scale_and_separate_buffers(gpu):
    S, H = 513, 2
    say(f"attention S={S} H={H} scale 0.05, separate Q/K/V buffers")
    qkv = qkv_buffer(S, H, 77, gpu)
    HD = H * D
    Q, K, V = (qkv[:, :HD].contiguous(), qkv[:, HD:2 * HD].contiguous(),
               qkv[:, 2 * HD:].contiguous())
    O = fsd.attention(Q, K, V, H, scale=0.05)
    ref = attention.attention_rows(Q.float().cpu().numpy(), K.float().cpu().numpy(),
                                   V.float().cpu().numpy(), heads=H, scale=0.05)
    ok, err = metrics.gemm_ok(O.float().cpu().numpy(), ref)
    say(f"  rel_l2 {err[0]:.3e} rel_max {err[1]:.3e}")
    assert ok, err


def test_attention_2k_grid_sampled_rows(gpu):
    """The 2K latent grid as one sequence (532,800 tokens), 24 heads of 128 (the
    stand-in width 3072): sampled query rows, each against all 532,800 keys."""
    from few_step_diffusion_amd import inputs
    S, H = inputs.WORKLOADS[4].tokens, 24
    say(f"attention 2K grid S={S} H={H}")
    qkv = qkv_buffer(S, H, 4242, gpu)
    rows = inputs.sample_rows(S, 12, seed=5)
    check(qkv, H, rows, "attention 2K sampled rows")


# ------------------------------------------------ attention inside the stand-in step
def _standin_oracle_layers(D, F, wid=4):
    import oracle
    from few_step_diffusion_amd import inputs
    layers = []
    for L in inputs.standin_layers(wid, D, F):
        Ab, Bb = oracle.merge_bf16([a.numpy() for a in L["A_list"]],
                                   [b.numpy() for b in L["B_list"]])
        layers.append({"W0": L["W0"].float().numpy(), "A": oracle.bf16_value(Ab).reshape(Ab.shape),
                       "B": oracle.bf16_value(Bb).reshape(Bb.shape)})
    E, P = inputs.standin_projections(wid, inputs.LATENT_C, D)
    return layers, E.float().numpy(), P.float().numpy()


def test_attention_step_every_token(gpu):
    """QKV -> attention -> O inside the three-step refine, every token of a
    4,133-token sequence (ragged against the 256-query and 64-key blocks) at
    width 256 (two heads of 128), against the fp64 oracle of the same step."""
    import oracle
    from few_step_diffusion_amd import inputs
    from few_step_diffusion_amd.refine import StandinRefiner
    M, Dm, Fm = 4133, 256, 512
    say(f"attention stand-in M={M} D={Dm} F={Fm}: every token, 3 steps")
    model = StandinRefiner(M, device=gpu, D=Dm, F=Fm, attention=True)
    u, eps = inputs.latent(4, tokens=M)
    z = model.refine(u.to(gpu), eps.to(gpu)).cpu().numpy()
    v = model.v.cpu().numpy()
    layers, E, P = _standin_oracle_layers(Dm, Fm)
    zh, vh = attention.standin_refine_attention(u.numpy(), eps.numpy(), E, P, layers,
                                                heads=Dm // D, sigmas=oracle.SIGMAS)
    e = metrics.token_error(z, zh[-1])
    ok, ev = metrics.gemm_ok(v, vh[-1])
    say(f"  final latent token err {e:.3e}; last velocity {ev}")
    assert e <= metrics.GEMM_TOL and ok
    # attention is exercised: the self-only stand-in's velocity differs far beyond the gate
    _, vs = oracle.standin_refine(u.numpy(), eps.numpy(), E, P, layers)
    assert metrics.row_errors(vs[-1], vh[-1])[0] > 5 * metrics.GEMM_TOL


def test_attention_step_2k_token_classes(gpu):
    """The attention step at the full 2K grid (532,800 tokens, 24 heads) on a
    latent with three distinct token values: a bulk class, a band of 1,800
    tokens in the middle and 666 tokens split between the two ends of the
    sequence (so the first and the last key blocks carry a class of their
    own).  Tokens of one class stay identical through the step, so the oracle
    computes the exact result from the three distinct rows with their
    multiplicities; every GPU token is compared with its class's row."""
    import oracle
    from few_step_diffusion_amd import inputs
    from few_step_diffusion_amd.refine import StandinRefiner
    M = inputs.WORKLOADS[4].tokens
    cls = np.zeros(M, np.int64)
    cls[200000:201800] = 1
    cls[:333] = 2
    cls[M - 333:] = 2
    mult = np.bincount(cls, minlength=3)
    say(f"attention stand-in at 2K, token classes {mult.tolist()}")
    u3, e3 = inputs.latent(4, tokens=3)
    u3[1] *= 2.0                                   # the band's keys stand out
    idx = torch.from_numpy(cls)
    u, eps = u3[idx].contiguous(), e3[idx].contiguous()
    model = StandinRefiner(M, device=gpu, attention=True)
    z = model.refine(u.to(gpu), eps.to(gpu))
    torch.cuda.synchronize()
    layers, E, P = _standin_oracle_layers(inputs.STANDIN_D, inputs.STANDIN_F)
    zh, _ = attention.standin_refine_attention(u3.numpy(), e3.numpy(), E, P, layers,
                                               heads=inputs.STANDIN_D // D,
                                               sigmas=oracle.SIGMAS, mult=mult)
    zg = z.cpu().numpy()
    for c in range(3):
        rows = zg[cls == c]
        spread = float(np.abs(rows - rows[0]).max() / np.abs(rows[0]).max())
        e = metrics.token_error(rows, np.tile(zh[-1][c], (rows.shape[0], 1)))
        say(f"  class {c} ({rows.shape[0]} tokens): token err {e:.3e}, spread {spread:.1e}")
        assert e <= metrics.GEMM_TOL
        assert spread <= 1e-6
    del model
    torch.cuda.empty_cache()
