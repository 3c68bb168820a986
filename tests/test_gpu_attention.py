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
