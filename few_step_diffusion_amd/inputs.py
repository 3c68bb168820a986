"""Seeded synthetic inputs shaped like the refiner's latents and layers.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic, imports neither the HIP binding nor the oracle, and
serves both sides.  Every tensor has a fixed seed:

    seed = 1000 * workload_id + 100 * layer + tensor_id

tensor ids: 1 u (upscaled latent, also x0), 2 eps (noise), 3 X (linear input
rows), 4 W0, 5-7 A_1..A_3, 8-10 B_1..B_3, 11 bias, 12 E (embed), 13 P (head).

Distributions: u, eps, X ~ N(0, 1); W0 ~ N(0, 0.02^2); A_i ~ N(0, 1/K);
B_i ~ N(0, 0.01^2); bias ~ N(0, 0.02^2); E ~ N(0, 1/C); P ~ N(0, 1/D).
Ranks 384 | 128 | 64 (merged 576): the refiner, Turbo and Sharp adapters of
"Open-H3-Regenerate-2K：MiniMax H3 的开源 4K 精修方案" (comfyui-wiki.com),
section "三个步如何完成工作".  Latent grids: 24 channels, 37 latent frames,
stride-16 target grids of "Open-H3-Regenerate-2K: High-Resolution Video
Refinement with Few-Step Diffusion" (agientry.com), sections "From any
low-resolution draft to native 4K" and "Why upscaling happens in latent space".

Host tensors come from numpy's PCG64; device tensors (large activations)
from torch's device generator seeded the same way.  bf16 operands are rounded
from fp32 once, by torch's round-to-nearest-even cast.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

RANKS = (384, 128, 64)
LATENT_C = 24

ID_U, ID_EPS, ID_X, ID_W0 = 1, 2, 3, 4
ID_A = (5, 6, 7)
ID_B = (8, 9, 10)
ID_BIAS, ID_E, ID_P = 11, 12, 13


def seed_of(workload: int, tensor_id: int, layer: int = 0) -> int:
    return 1000 * workload + 100 * layer + tensor_id


def normal(shape, std, seed, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """N(0, std^2) tensor.  Host: numpy PCG64.  Device: torch generator."""
    shape = tuple(int(s) for s in shape)
    dev = torch.device(device)
    if dev.type == "cpu":
        g = np.random.Generator(np.random.PCG64(seed))
        a = g.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        t = torch.from_numpy(a)
    else:
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        t = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
    return t if dtype == torch.float32 else t.to(dtype)


@dataclass
class Workload:
    """One of the five synthetic workloads (latent grid + linear shapes)."""
    wid: int
    name: str
    frames: int
    height: int
    width: int
    linears: list = field(default_factory=list)   # (label, K, N, swiglu)
    chunks: int = 1

    @property
    def tokens(self) -> int:
        return self.frames * self.height * self.width

    @property
    def latent_elems(self) -> int:
        return LATENT_C * self.tokens


WORKLOADS = {
    0: Workload(0, "tiny 24x5x12x20, LoRA 1024x1024", 5, 12, 20, [("linear", 1024, 1024, False)]),
    1: Workload(1, "768P grid 24x37x48x84, LoRA 3072x3072", 37, 48, 84,
                [("linear", 3072, 3072, False)]),
    2: Workload(2, "2K grid 24x37x90x160, QKV 3072->9216 and O 3072->3072", 37, 90, 160,
                [("qkv", 3072, 9216, False), ("o", 3072, 3072, False)]),
    3: Workload(3, "4K grid 24x37x135x240 in 4 chunks, gate/up 3072->2x8192 SwiGLU, "
                   "down 8192->3072", 37, 135, 240,
                [("gate_up", 3072, 16384, True), ("down", 8192, 3072, False)], chunks=4),
    4: Workload(4, "2K three-step sweep, 4-layer LoRA stand-in d=3072 ffn=8192 r=576",
                37, 90, 160, [("qkv", 3072, 9216, False), ("o", 3072, 3072, False),
                              ("gate_up", 3072, 16384, True), ("down", 8192, 3072, False)]),
}

STANDIN_D = 3072
STANDIN_F = 8192


def latent(wid: int, tokens: int | None = None):
    """(u, eps): fp32 [tokens, 24] channel-last latent rows, N(0, 1)."""
    T = WORKLOADS[wid].tokens if tokens is None else tokens
    u = normal((T, LATENT_C), 1.0, seed_of(wid, ID_U))
    e = normal((T, LATENT_C), 1.0, seed_of(wid, ID_EPS))
    return u, e


def activations(wid: int, M: int, K: int, device="cpu", layer: int = 0) -> torch.Tensor:
    """X ~ N(0, 1) rounded to bf16, [M, K]."""
    return normal((M, K), 1.0, seed_of(wid, ID_X, layer), device=device, dtype=torch.bfloat16)


def adapters(wid: int, K: int, N: int, layer: int = 0, ranks=RANKS):
    """Three LoRA adapters in fp32 storage: A_i [r_i, K] ~ N(0, 1/K), B_i [N, r_i] ~ N(0, 1e-4)."""
    A = [normal((r, K), K ** -0.5, seed_of(wid, ID_A[i], layer)) for i, r in enumerate(ranks)]
    B = [normal((N, r), 0.01, seed_of(wid, ID_B[i], layer)) for i, r in enumerate(ranks)]
    return A, B


def base_weight(wid: int, K: int, N: int, layer: int = 0) -> torch.Tensor:
    """W0 ~ N(0, 0.02^2) rounded to bf16, [N, K] (out_features x in_features)."""
    return normal((N, K), 0.02, seed_of(wid, ID_W0, layer), dtype=torch.bfloat16)


def bias(wid: int, N: int, layer: int = 0) -> torch.Tensor:
    return normal((N,), 0.02, seed_of(wid, ID_BIAS, layer))


def standin_projections(wid: int = 4, C: int = LATENT_C, D: int = STANDIN_D):
    """E [D, C] ~ N(0, 1/C) and P [C, D] ~ N(0, 1/D), both rounded to bf16."""
    E = normal((D, C), C ** -0.5, seed_of(wid, ID_E), dtype=torch.bfloat16)
    P = normal((C, D), D ** -0.5, seed_of(wid, ID_P), dtype=torch.bfloat16)
    return E, P


def standin_layers(wid: int = 4, D: int = STANDIN_D, F: int = STANDIN_F, ranks=RANKS):
    """Four layers (qkv, o, gate/up, down): dicts with W0 (bf16), A_list, B_list (fp32)."""
    shapes = [(D, 3 * D), (D, D), (D, 2 * F), (F, D)]   # (K, N)
    out = []
    for li, (K, N) in enumerate(shapes, start=1):
        A, B = adapters(wid, K, N, layer=li, ranks=ranks)
        out.append({"W0": base_weight(wid, K, N, layer=li), "A_list": A, "B_list": B,
                    "K": K, "N": N})
    return out


def sample_rows(M: int, count: int, seed: int, tile: int = 256) -> np.ndarray:
    """A fixed row sample: first and last rows, rows on either side of every
    `tile` boundary while the budget lasts, the rest uniform at random."""
    if M <= count:
        return np.arange(M, dtype=np.int64)
    rows = set(range(min(4, M))) | set(range(max(0, M - 4), M))
    b = tile
    while b < M and len(rows) < count // 2:
        rows.update((b - 1, b))
        b += tile * max(1, (M // tile) // max(1, count // 4))
    g = np.random.Generator(np.random.PCG64(seed))
    while len(rows) < count:
        rows.add(int(g.integers(0, M)))
    return np.array(sorted(rows), dtype=np.int64)
