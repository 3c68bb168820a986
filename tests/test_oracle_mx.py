"""Pins of the MXFP8 oracle (oracle/mx.py) against the OCP MX v1.0 format facts,
an independent library conversion (torch's float8_e4m3fn cast) and closed forms."""
import math

import numpy as np
import pytest
import torch

from oracle import mx


def test_e4m3_code_table():
    finite = [b for b in range(256) if (b & 0x7F) != 0x7F]
    vals = [mx.e4m3_value(b) for b in finite]
    assert max(vals) == 448.0 and mx.e4m3_bits(448.0) == 0x7E       # largest finite E4M3
    assert mx.e4m3_value(0x01) == 2.0 ** -9                          # smallest subnormal
    assert mx.e4m3_value(0x08) == 2.0 ** -6                          # smallest normal
    assert mx.e4m3_value(0x38) == 1.0
    for b in finite:                                                 # every code round-trips
        v = mx.e4m3_value(b)
        assert mx.e4m3_round(v) == v
        if v != 0.0:
            assert mx.e4m3_bits(v) == b


def test_e4m3_ties_go_to_even():
    assert mx.e4m3_round(1.0 + 1 / 16) == 1.0          # halfway between 1 and 1.125
    assert mx.e4m3_round(1.0 + 3 / 16) == 1.25         # halfway between 1.125 and 1.25
    assert mx.e4m3_round(-(1.0 + 3 / 16)) == -1.25
    assert mx.e4m3_round(2.0 ** -10) == 0.0            # half the smallest subnormal -> 0 (even)
    assert mx.e4m3_round(3 * 2.0 ** -10) == 2.0 ** -8  # 1.5 quanta -> 2 quanta


def test_e4m3_saturates():
    assert mx.e4m3_round(460.0) == 448.0
    assert mx.e4m3_round(1e6) == 448.0
    assert mx.e4m3_round(-500.0) == -448.0


def test_e4m3_matches_torch_cast_in_range():
    """torch's float8_e4m3fn cast (an independent implementation, nearest-even) agrees on
    every value inside the finite range, including subnormals and ties."""
    rng = np.random.default_rng(7)
    ys = np.concatenate([rng.standard_normal(4000) * 40.0,
                         rng.standard_normal(2000) * 2.0 ** -7,
                         np.array([mx.e4m3_value(b) for b in range(0, 0x7E)]) * (1 + 1 / 16)])
    ys = ys[np.abs(ys) < 448.0]
    t = torch.from_numpy(ys).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    o = np.array([mx.e4m3_round(float(y)) for y in ys])
    assert np.array_equal(t, o)


def test_block_exponent_and_scaling():
    assert mx.block_exponent([1.0] + [0.0] * 31) == -8          # amax 1 -> X = 2^-8, 1/X = 256
    assert mx.block_exponent([0.0] * 32) == -127
    assert mx.block_exponent([3.0, -300.0]) == math.floor(math.log2(300.0)) - 8
    q, s = mx.quantize_rows(np.array([[1.0] + [0.5] * 31]))
    assert q.shape == (1, 128) and s.shape == (1, 4)
    assert s[0, 0] == 127 - 8 and s[0, 1] == 127                 # padded blocks: scale 1
    assert mx.e4m3_value(int(q[0, 0])) == 256.0 and mx.e4m3_value(int(q[0, 1])) == 128.0
    assert np.all(q[0, 32:] == 0)


def test_quantization_error_bound():
    """Per element: half a unit in the last place of E4M3 (2^-4 relative) for normal
    results, the subnormal quantum below them, and the 448..512 clip of the top binade."""
    rng = np.random.default_rng(11)
    X = rng.standard_normal((6, 96)) * np.exp(rng.standard_normal((6, 1)) * 3)
    q, s = mx.quantize_rows(X)
    D = mx.dequantize_rows(q, s, 96)
    for i in range(6):
        for k in range(96):
            X_scale = 2.0 ** (int(s[i, k // 32]) - 127)
            y = X[i, k] / X_scale
            if abs(y) > 448.0:
                bound = (abs(y) - 448.0) * X_scale
            else:
                bound = max(abs(X[i, k]) * 2.0 ** -4, 2.0 ** -10 * X_scale)
            assert abs(D[i, k] - X[i, k]) <= bound * (1 + 1e-12), (i, k)


def _awkward_rows():
    """Rows over many binades with zeros, huge and tiny rows, E4M3 ties, saturating
    values, subnormal results and signed zeros."""
    rng = np.random.default_rng(5)
    X = rng.standard_normal((9, 160)) * np.exp(rng.standard_normal((9, 1)) * 4.0)
    X[0] = 0.0
    X[1] *= 1e36
    X[2] *= 1e-36
    ties = [1.0625, 1.1875, 1.3125, 1.4375, 1.5625, 1.6875, 1.8125, 1.875, 1.9375]
    X[3, :32] = 0.0
    X[3, :9] = ties
    X[3, 9:18] = [-t for t in ties]
    X[4, :32] = -0.0
    X[4, 0] = 1.0
    X[4, 1:8] = [-2.0 ** -20, 2.0 ** -17, -2.0 ** -16.5, 2.0 ** -14.9, 3.0 * 2.0 ** -18,
                 -5.0 * 2.0 ** -18, 2.0 ** -18]                  # subnormal and flushed results
    X[5, :32] = np.linspace(-1.0, 1.0, 32)
    X[5, 32:64] = 0.0
    X[5, 32] = -2.0 ** -140                                      # a tiny-amax block
    return X


def test_array_form_matches_element_loops():
    X = _awkward_rows()
    q, s = mx.quantize_rows(X)
    qn, sn = mx.quantize_rows_np(X)
    assert np.array_equal(q, qn) and np.array_equal(s, sn)
    assert np.array_equal(mx.dequantize_rows(q, s, 160), mx.dequantize_rows_np(q, s, 160))
    # every byte pattern but the NaNs decodes the same way
    codes = np.array([[b for b in range(256) if (b & 0x7F) != 0x7F][:224]], np.uint8)
    sc = np.array([[120, 127, 134, 2, 250, 127, 64]], np.uint8)
    assert np.array_equal(mx.dequantize_rows(codes, sc, 224),
                          mx.dequantize_rows_np(codes, sc, 224))


def test_bf16_round_matches_the_c_oracle():
    import oracle
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(2000) * np.exp(rng.standard_normal(2000) * 6),
                        # exact bf16 ties (even and odd) and their neighbours
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8),
                                  1.0 + 2.0 ** -8 + 2.0 ** -20, 0.0, -0.0, 3.0e38])])
    ref = oracle.bf16_value(oracle.bf16_bits(x.astype(np.float32))).astype(np.float64)
    got = mx.bf16_round_np(x)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def _tiny_standin(seed=3, T=3, C=4, D=32, F=64, r=32):
    rng = np.random.default_rng(seed)
    bf = mx.bf16_round_np
    layers = []
    for K, N in [(D, 3 * D), (D, D), (D, 2 * F), (F, D)]:
        layers.append({"W0": bf(rng.standard_normal((N, K)) * 0.2),
                       "A": bf(rng.standard_normal((r, K)) / math.sqrt(K)),
                       "B": bf(rng.standard_normal((N, r)) * 0.1), "scale": 0.5})
    E = bf(rng.standard_normal((D, C)))
    P = bf(rng.standard_normal((C, D)) * 0.05)
    z = rng.standard_normal((T, C))
    return z, E, P, layers


def test_mx_standin_velocity_by_element_loops():
    """The array-form MXFP8 stand-in against the same data flow written with the
    element-loop quantizer and explicit loops for every product (tiny shapes)."""
    z, E, P, layers = _tiny_standin()
    T, C = z.shape
    D = E.shape[0]
    F = layers[3]["W0"].shape[1]
    bf = mx.bf16_round_np

    def qd(X):                                   # element-loop quantize + dequantize
        q, s = mx.quantize_rows(X)
        return mx.dequantize_rows(q, s, X.shape[1])

    def matT(X, W):                              # X·Wᵀ by loops
        out = np.zeros((X.shape[0], W.shape[0]))
        for i in range(X.shape[0]):
            for j in range(W.shape[0]):
                out[i, j] = sum(X[i, k] * W[j, k] for k in range(X.shape[1]))
        return out

    def lin(X, L):
        Xd = qd(X)
        Td = qd(bf(L["scale"] * matT(Xd, qd(L["A"]))))
        return matT(Xd, qd(L["W0"])) + matT(Td, qd(L["B"]))

    h = bf(matT(z, E))
    qkv = bf(lin(h, layers[0]))
    h = bf(lin(qkv[:, 2 * D:], layers[1]) + h)
    y = lin(h, layers[2])
    g = np.zeros((T, F))
    for i in range(T):
        for j in range(F):
            a, b = y[i, j], y[i, F + j]
            g[i, j] = a / (1.0 + math.exp(-a)) * b
    h = bf(lin(bf(g), layers[3]) + h)
    v_ref = matT(h, P)
    v = mx.standin_velocity_mx(z, E, P, mx.standin_mx_weights(layers))
    assert np.allclose(v, v_ref, rtol=1e-12, atol=1e-12)


def test_mx_standin_velocity_within_the_mxfp8_budget_of_the_exact_one():
    """Against the exact fp64 stand-in (the C oracle): quantizing every linear's
    operands to MXFP8 (about 3% RMS per element, four chained linears and a
    SwiGLU at this small width) moves the velocity by roughly 10-15% of its
    norm, never by nothing, while a gross slip - the LoRA path dropped (half the
    output here), a wrong slice or residual - moves it by far more."""
    import oracle
    z, E, P, layers = _tiny_standin(seed=4, T=64, D=64, F=128)
    layers = [dict(L, scale=1.0, B=mx.bf16_round_np(L["B"] * 2)) for L in layers]
    v = oracle.standin_velocity(z, E, P, layers)
    v_mx = mx.standin_velocity_mx(z, E, P, mx.standin_mx_weights(layers))
    err = np.linalg.norm(v_mx - v) / np.linalg.norm(v)
    assert 0.01 < err < 0.25, err
    no_lora = [dict(L, scale=0.0) for L in layers]
    v_drop = mx.standin_velocity_mx(z, E, P, mx.standin_mx_weights(no_lora))
    assert np.linalg.norm(v_drop - v) / np.linalg.norm(v) > 0.5
