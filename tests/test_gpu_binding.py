"""The Python binding checks every tensor's extent against the sizes it passes
to the C ABI, before any launch: a wrongly sized output, workspace, scale array
or operand raises ValueError (the library itself sees only pointers and sizes,
so such a buffer would otherwise be read or written out of bounds)."""
import pytest
import torch

import few_step_diffusion_amd as fsd

pytestmark = pytest.mark.gpu

bf = torch.bfloat16


def _t(shape, dtype=bf, dev="cuda:0"):
    return torch.zeros(shape, dtype=dtype, device=dev)


def test_lora_linear_shapes(gpu):
    M, K, N, r = 300, 256, 320, 64
    X, W0, A, B = _t((M, K)), _t((N, K)), _t((r, K)), _t((N, r))
    bad = [
        dict(out=_t((M, N - 8))),                       # output too narrow
        dict(out=_t((M - 1, N))),                       # output too short
        dict(residual=_t((M, N + 8))),
        dict(bias=torch.zeros(N - 1, device=gpu)),
        dict(epilogue="swiglu", out=_t((M, N))),        # SwiGLU writes N/2 columns
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            fsd.lora_linear(X, W0, A, B, **kw)
    with pytest.raises(ValueError):
        fsd.lora_linear(X, _t((N, K + 8))[:, :K], A, B)   # W0 must be contiguous [N, K]
    with pytest.raises(ValueError):
        fsd.lora_linear(X, W0, _t((r, K - 8)), B)
    with pytest.raises(ValueError):
        fsd.lora_linear(X, W0, A, _t((N, r + 8)))
    with pytest.raises(ValueError):
        fsd.lora_up(X, W0, _t((M, r - 8)), B)
    with pytest.raises(ValueError):
        fsd.lora_down(X, A, T=_t((M + 1, r)))
    torch.cuda.synchronize()


def test_standin_and_mx_shapes(gpu):
    M, C, D = 100, 24, 256
    z = torch.zeros((M, C), device=gpu)
    E, P = _t((D, C)), _t((C, D))
    with pytest.raises(ValueError):
        fsd.token_embed(z, E, out=_t((M, D - 8)))
    with pytest.raises(ValueError):
        fsd.token_head(_t((M, D)), P, out=torch.zeros((M, C - 1), device=gpu))
    with pytest.raises(ValueError):
        fsd.token_head_euler(_t((M, D)), P, torch.zeros((M - 1, C), device=gpu), 0.9, 0.8)
    X = _t((M, 256))
    with pytest.raises(ValueError):
        fsd.mx_quantize(X, Q=torch.zeros((M, 128), dtype=torch.uint8, device=gpu))
    with pytest.raises(ValueError):
        fsd.mx_quantize(X, S=torch.zeros(16, dtype=torch.uint8, device=gpu))
    with pytest.raises(ValueError):
        fsd.attention(_t((64, 256)), _t((64, 256)), _t((64, 256)), 2, out=_t((64, 128)))
    torch.cuda.synchronize()
