"""Pins of the attention oracle (oracle/attention.py) against closed forms,
invariances and an element-by-element formulation on tiny shapes."""
import math

import numpy as np

from oracle import attention


def _qkv(S, H, D, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((S, H * D)), rng.standard_normal((S, H * D)),
            rng.standard_normal((S, H * D)))


def test_equal_keys_average_the_values():
    """Identical keys give every key the same weight: O is the mean of V."""
    Q, _, V = _qkv(7, 2, 8, 1)
    K = np.tile(np.random.default_rng(2).standard_normal((1, 16)), (7, 1))
    O = attention.attention_rows(Q, K, V, heads=2)
    assert np.allclose(O, np.tile(V.mean(axis=0), (7, 1)), rtol=0, atol=1e-13)


def test_one_dominant_key_selects_its_value():
    S, D = 5, 4
    K = np.zeros((S, D))
    K[3] = [30.0, 0, 0, 0]
    Q = np.tile([[1.0, 0, 0, 0]], (2, 1)) * math.sqrt(D)    # logit 30 against 0
    V = np.arange(S * D, dtype=np.float64).reshape(S, D)
    O = attention.attention_rows(Q, K, V, heads=1)
    w = math.exp(30.0) / (math.exp(30.0) + 4.0)               # closed form of the weights
    expect = w * V[3] + (1 - w) / 4 * (V.sum(axis=0) - V[3])
    assert np.allclose(O, np.tile(expect, (2, 1)), rtol=1e-14, atol=0)


def test_two_keys_closed_form_pins_the_scale():
    """Two keys with logits a and b: weights e^a/(e^a+e^b); the 1/sqrt(D) scale
    and a custom scale are both checked."""
    D = 16
    q = np.zeros((1, D)); q[0, 0] = 2.0
    K = np.zeros((2, D)); K[0, 0] = 3.0; K[1, 0] = -1.0
    V = np.array([[1.0] * D, [-2.0] * D])
    for scale in (None, 0.7):
        s = 1 / math.sqrt(D) if scale is None else scale
        a, b = 6.0 * s, -2.0 * s
        w0 = 1 / (1 + math.exp(b - a))
        O = attention.attention_rows(q, K, V, heads=1, scale=scale)
        assert np.allclose(O, w0 * V[0] + (1 - w0) * V[1], rtol=1e-14, atol=1e-15)


def test_key_permutation_invariance_and_row_subset():
    Q, K, V = _qkv(40, 3, 16, 3)
    perm = np.random.default_rng(4).permutation(40)
    O = attention.attention_rows(Q, K, V, heads=3)
    assert np.allclose(O, attention.attention_rows(Q, K[perm], V[perm], heads=3),
                       rtol=1e-12, atol=1e-13)
    rows = np.array([0, 7, 39])
    assert np.allclose(attention.attention_rows(Q, K, V, heads=3, rows=rows), O[rows],
                       rtol=0, atol=0)


def test_heads_are_independent_and_match_element_loops():
    """Each head's output depends on its own columns only, and equals the
    definition evaluated with explicit loops (exp of the raw logits, no shift)."""
    S, H, D = 6, 2, 4
    Q, K, V = _qkv(S, H, D, 5)
    O = attention.attention_rows(Q, K, V, heads=H)
    ref = np.zeros((S, H * D))
    for h in range(H):
        for i in range(S):
            logits = [sum(Q[i, h * D + d] * K[j, h * D + d] for d in range(D)) / math.sqrt(D)
                      for j in range(S)]
            den = sum(math.exp(x) for x in logits)
            for d in range(D):
                ref[i, h * D + d] = sum(math.exp(logits[j]) * V[j, h * D + d]
                                        for j in range(S)) / den
    assert np.allclose(O, ref, rtol=1e-12, atol=1e-14)
    K2 = K.copy()
    K2[:, D:] = 0.0                                            # change head 1 only
    O2 = attention.attention_rows(Q, K2, V, heads=H)
    assert np.array_equal(O2[:, :D], O[:, :D]) and not np.allclose(O2[:, D:], O[:, D:])


# ------------------------------------------------ key multiplicities, stand-in
def test_key_multiplicity_equals_repeated_keys():
    """A key row with multiplicity m is the same as m copies of that row."""
    Q, K, V = _qkv(5, 2, 8, 11)
    m = np.array([1, 3, 1, 2, 5])
    rep = np.repeat(np.arange(5), m)
    O_rep = attention.attention_rows(Q, K[rep], V[rep], heads=2)
    O_mult = attention.attention_rows(Q, K, V, heads=2, key_mult=m)
    assert np.allclose(O_mult, O_rep, rtol=1e-13, atol=1e-14)
    assert np.allclose(attention.attention_rows(Q, K, V, heads=2, key_mult=np.ones(5)),
                       attention.attention_rows(Q, K, V, heads=2), rtol=0, atol=0)


def _tiny_standin(T=6, C=4, D=256, F=64, seed=3):
    import oracle
    from few_step_diffusion_amd import inputs
    ranks = (16, 8, 8)
    layers = []
    for L in inputs.standin_layers(4, D, F, ranks):
        Ab, Bb = oracle.merge_bf16([a.numpy() for a in L["A_list"]],
                                   [b.numpy() for b in L["B_list"]])
        layers.append({"W0": L["W0"].float().numpy(), "A": oracle.bf16_value(Ab).reshape(Ab.shape),
                       "B": oracle.bf16_value(Bb).reshape(Bb.shape)})
    E, P = inputs.standin_projections(4, C, D)
    rng = np.random.default_rng(seed)
    x0 = rng.standard_normal((T, C)).astype(np.float32)
    eps = rng.standard_normal((T, C)).astype(np.float32)
    return x0, eps, E.float().numpy(), P.float().numpy(), layers


def test_attention_standin_with_identical_tokens_is_the_self_only_standin():
    """Identical tokens attend to identical keys: every token's attention output
    is its own V, which is the self-only stand-in of the C oracle."""
    import oracle
    x0, eps, E, P, layers = _tiny_standin()
    x0 = np.tile(x0[:1], (5, 1))
    eps = np.tile(eps[:1], (5, 1))
    z_att, v_att = attention.standin_refine_attention(x0, eps, E, P, layers, heads=2,
                                                      sigmas=oracle.SIGMAS)
    z_self, v_self = oracle.standin_refine(x0, eps, E, P, layers)
    assert np.allclose(z_att, z_self, rtol=1e-10, atol=1e-12)
    assert np.allclose(v_att, v_self, rtol=1e-10, atol=1e-12)


def test_attention_standin_token_permutation_and_multiplicities():
    """Permuting the tokens permutes the result; a token class given once with
    multiplicity m equals the class repeated m times."""
    import oracle
    x0, eps, E, P, layers = _tiny_standin(T=4)
    perm = np.array([2, 0, 3, 1])
    za, _ = attention.standin_refine_attention(x0, eps, E, P, layers, 2, oracle.SIGMAS)
    zp, _ = attention.standin_refine_attention(x0[perm], eps[perm], E, P, layers, 2,
                                               oracle.SIGMAS)
    assert np.allclose(zp, za[:, perm], rtol=1e-12, atol=1e-13)
    m = np.array([3, 1, 2, 4])
    rep = np.repeat(np.arange(4), m)
    zr, _ = attention.standin_refine_attention(x0[rep], eps[rep], E, P, layers, 2,
                                               oracle.SIGMAS)
    zm, _ = attention.standin_refine_attention(x0, eps, E, P, layers, 2, oracle.SIGMAS, mult=m)
    assert np.allclose(zm[:, rep], zr, rtol=1e-11, atol=1e-12)
    # attention matters here: the self-only stand-in differs
    zs, _ = oracle.standin_refine(x0, eps, E, P, layers)
    assert not np.allclose(zs, za, rtol=1e-3, atol=1e-3)
