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


def attention_rows(Q, K, V, heads, rows=None, scale=None):
    """O[rows] for Q, K, V of shape [S, heads·D] (head h in columns h·D .. h·D+D-1).

    Returns float64 [len(rows), heads·D].
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    S, HD = K.shape
    D = HD // heads
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rows = np.arange(Q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), HD), np.float64)
    for h in range(heads):
        cols = slice(h * D, (h + 1) * D)
        logits = (Q[rows, cols] @ K[:, cols].T) * scale         # [rows, S]
        logits -= logits.max(axis=1, keepdims=True)
        w = np.exp(logits)
        w /= w.sum(axis=1, keepdims=True)
        out[:, cols] = w @ V[:, cols]
    return out
