"""fp64 reference of dense softmax attention — TEST INFRASTRUCTURE ONLY.

The pages' baseline refine path runs the transformer's attention densely in bf16
([EN] "Open-H3-Regenerate-2K: High-Resolution Video Refinement with Few-Step
Diffusion", section "Where the 3.9x speedup comes from": the dense-BF16-attention
baseline row and the Sol-Attn row).  They name the operation only; this is the
textbook scaled dot-product attention (Vaswani et al. 2017), per head:

    O_h = softmax(Q_h · K_hᵀ · scale) · V_h,    scale = 1/sqrt(D) by default,

the softmax taken over all keys of the sequence for each query row.  The row
maximum is subtracted before exponentiating, which leaves the softmax unchanged.
Inputs are the exact values the GPU receives, widened to float64.
"""
from __future__ import annotations

import math

import numpy as np


def attention_rows(Q, K, V, heads, rows=None, scale=None, key_mult=None):
    """O[rows] for Q, K, V of shape [S, heads·D] (head h in columns h·D .. h·D+D-1).

    key_mult: optional multiplicities [S] of the key/value rows (row j stands for
    key_mult[j] identical tokens), i.e. weights m_j·exp(logit) in both softmax
    sums; None is multiplicity 1 everywhere.  Returns float64 [len(rows), heads·D].
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    S, HD = K.shape
    D = HD // heads
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rows = np.arange(Q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    m = None if key_mult is None else np.asarray(key_mult, dtype=np.float64)
    out = np.empty((len(rows), HD), np.float64)
    for h in range(heads):
        cols = slice(h * D, (h + 1) * D)
        logits = (Q[rows, cols] @ K[:, cols].T) * scale         # [rows, S]
        logits -= logits.max(axis=1, keepdims=True)
        w = np.exp(logits)
        if m is not None:
            w *= m[None, :]
        w /= w.sum(axis=1, keepdims=True)
        out[:, cols] = w @ V[:, cols]
    return out


def standin_refine_attention(x0, eps, E, P, layers, heads, sigmas, mult=None, scale=None,
                             nthreads=0):
    """The refine with the velocity stand-in whose QKV and O linears have dense
    attention between them, over all T tokens as one sequence (the DiT view of
    the latent):

        x = z·Eᵀ;  [q | k | v] = L_qkv(x);  a = attention(q, k, v)  (per head);
        h = x + L_o(a);  h = h + L_down(SwiGLU(L_gu(h)));  velocity = h·Pᵀ,

    then renoise at sigmas[0] and one Euler step per sigma pair, all in float64
    (no intermediate rounding).  The linears are the C oracle's (lora_linear_drows);
    embed, head, SwiGLU and attention are the textbook formulas above.
    mult: optional token multiplicities [T]: row j stands for mult[j] identical
    tokens (their keys and values enter the softmax with that weight), so a
    latent with few distinct tokens is computed exactly from its distinct rows.
    layers: 4 dicts (W0, A, B, optional scale) for qkv, o, gate/up, down.
    Returns (z_hist [nsig, T, C], v_hist [nsig-1, T, C])."""
    from . import euler_step, lora_linear_drows, renoise
    E = np.asarray(E, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    D = E.shape[0]
    F = np.asarray(layers[3]["W0"]).shape[1]

    def lin(X, L):
        return lora_linear_drows(X, L["W0"], L.get("A"), L.get("B"), scale=L.get("scale", 1.0),
                                 nthreads=nthreads)

    def velocity(z):
        x = z @ E.T
        qkv = lin(x, layers[0])
        a = attention_rows(qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:3 * D], heads,
                           scale=scale, key_mult=mult)
        h = x + lin(a, layers[1])
        y = lin(h, layers[2])
        g = y[:, :F] / (1.0 + np.exp(-y[:, :F])) * y[:, F:]
        h = h + lin(g, layers[3])
        return h @ P.T

    z = renoise(x0, eps, sigmas[0])
    zs, vs = [z], []
    for k in range(len(sigmas) - 1):
        v = velocity(z)
        z = euler_step(z, v, sigmas[k], sigmas[k + 1])
        zs.append(z)
        vs.append(v)
    return np.stack(zs), np.stack(vs)
