"""GPU parity of the MXFP8 path against the fp64 MX oracle (oracle/mx.py).

Quantization is byte work: elements and scales must match the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import few_step_diffusion_amd as fsd
from oracle import mx

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[case] {msg}", flush=True)


def mx_rows(M, K, seed):
    """bf16 rows over many binades, plus an all-zero row, huge and tiny rows and a row
    of exact E4M3 rounding ties."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)) * 4.0)
    if M > 3:
        X[0] = 0.0
        X[1] *= 1e36
        X[2] *= 1e-36
    if M > 4 and K >= 32:
        # with block max 1.9375 the scale is 2^-8: these land halfway between E4M3
        # values of the top binade (272, 304, ...) or past 448 (saturation)
        ties = [1.0625, 1.1875, 1.3125, 1.4375, 1.5625, 1.6875, 1.8125, 1.875, 1.9375]
        X[3, :32] = 0.0
        X[3, :len(ties)] = ties
        X[3, len(ties):2 * len(ties)] = [-t for t in ties]
    return torch.from_numpy(X).to(torch.bfloat16)


def scales_by_row(S, M, K):
    """Rows x blocks view of the step-major scale array [Kp/128][Mp][4]."""
    Kp = fsd.mx_padded_k(K)
    Mp = (M + 255) // 256 * 256
    t = S.cpu().numpy().reshape(Kp // 128, Mp, 4)
    return t.transpose(1, 0, 2).reshape(Mp, Kp // 32)


@pytest.mark.parametrize("M,K", [(1, 32), (5, 96), (300, 576), (8, 3072)])
def test_mx_quantize_bit_exact(gpu, M, K):
    say(f"mx quantize M={M} K={K}")
    Xb = mx_rows(M, K, seed=M * 1000 + K)
    Q, S = fsd.mx_quantize(Xb.to(gpu))
    q_ref, s_ref = mx.quantize_rows(Xb.float().numpy())
    Kp = fsd.mx_padded_k(K)
    assert Q.shape == (M, Kp)
    q = Q.cpu().numpy()
    bad = np.argwhere(q != q_ref)
    assert bad.size == 0, (len(bad), bad[:5], q[tuple(bad[0])], q_ref[tuple(bad[0])])
    s_rows = scales_by_row(S, M, K)
    assert np.array_equal(s_rows[:M], s_ref)
    assert np.all(s_rows[M:] == 127)
