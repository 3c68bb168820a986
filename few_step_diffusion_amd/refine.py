"""The three-step refine loop over a 2K latent with a synthetic 4-layer velocity
stand-in whose linears all carry the merged rank-576 LoRA.

Method ("Open-H3-Regenerate-2K: High-Resolution Video Refinement with Few-Step
Diffusion", agientry.com, section "Three steps instead of dozens"): re-noise
the upscaled latent to sigma_0 = 0.909, then one velocity evaluation and one
Euler update per step along 0.909 -> 0.857 -> 0.667 -> 0, classifier-free
guidance off.  The real transformer's widths and weights are not available;
the stand-in per token is

    x = z·Eᵀ;  q = L_qkv(x);  h = x + L_o(q[:, 2D:3D]);
    h = h + L_down(SwiGLU(L_gu(h)));  v = h·Pᵀ

with every L_* the LoRA-fused linear.  Every call below is one HIP kernel of
libfsd.so (through the ctypes binding); torch only allocates device memory
and supplies the stream.
"""
from __future__ import annotations

import torch

from . import binding as fsd
from . import inputs
from .schedules import REFINE as SIGMAS


class StandinRefiner:
    """Device-resident weights and activation buffers for M tokens."""

    LAYER_NAMES = ("qkv", "o", "gate_up", "down")

    def __init__(self, M: int, device="cuda:0", wid: int = 4, D: int = inputs.STANDIN_D,
                 F: int = inputs.STANDIN_F, ranks=inputs.RANKS, C: int = inputs.LATENT_C,
                 scale: float = 1.0, mx: bool = False):
        """mx: run the four linears as MXFP8 GEMMs.  The bf16 weights are quantized
        once here; each linear quantizes its bf16 input and its bf16 LoRA down output,
        and the gate/up GEMM hands SwiGLU's output to the down projection already
        quantized."""
        dev = torch.device(device)
        self.M, self.D, self.F, self.C, self.dev = M, D, F, C, dev
        self.R = sum(ranks)
        self.scale = scale
        self.mx = mx
        self.layers = []
        for L in inputs.standin_layers(wid, D, F, ranks):
            A, B = fsd.lora_merge([a.to(dev) for a in L["A_list"]],
                                  [b.to(dev) for b in L["B_list"]])
            layer = {"W0": L["W0"].to(dev), "A": A, "B": B, "K": L["K"], "N": L["N"]}
            if mx:
                layer["W0q"] = fsd.mx_quantize(layer.pop("W0"))
                layer["Aq"] = fsd.mx_quantize(layer.pop("A"))
                layer["Bq"] = fsd.mx_quantize(layer.pop("B"))
            self.layers.append(layer)
        E, P = inputs.standin_projections(wid, C, D)
        self.E, self.P = E.to(dev), P.to(dev)
        bf = torch.bfloat16
        self.h = torch.empty((M, D), dtype=bf, device=dev)            # residual stream
        self.qkv = torch.empty((M, 3 * D), dtype=bf, device=dev)
        self.g = torch.empty((M, F), dtype=bf, device=dev)            # SwiGLU output
        self.T = torch.empty((M, self.R), dtype=bf, device=dev)      # LoRA down output
        self.v = torch.empty((M, C), dtype=torch.float32, device=dev)
        self.z = torch.empty((M, C), dtype=torch.float32, device=dev)
        if mx:
            u8 = torch.uint8
            mxbuf = lambda K: (torch.empty((M, fsd.mx_padded_k(K)), dtype=u8, device=dev),
                               torch.empty(max(fsd.mx_scale_bytes(M, K), 4), dtype=u8,
                                           device=dev))
            self.hq = mxbuf(D)           # linear inputs: h, then V
            self.vq = mxbuf(D)
            self.gq = mxbuf(F)           # SwiGLU output, quantized by the gate/up GEMM
            self.tq = mxbuf(self.R)      # LoRA down output
            del self.g
        self.events = None

    # one LoRA linear = phase A + phase B (two kernels)
    def _linear(self, idx, X, out, residual=None, epilogue=fsd.EPI_NONE):
        L = self.layers[idx]
        T = self.T[: X.shape[0]]
        self._mark(f"{self.LAYER_NAMES[idx]}.down")
        fsd.lora_down(X, L["A"], self.scale, T)
        self._mark(f"{self.LAYER_NAMES[idx]}.up")
        fsd.lora_up(X, L["W0"], T, L["B"], residual=residual, epilogue=epilogue, out=out)

    def _mark(self, name):
        if self.events is not None:
            ev = torch.cuda.Event(enable_timing=True)
            ev.record()
            self.events.append((name, ev))

    # one MXFP8 LoRA linear: phase A, quantize T, phase B (SwiGLU -> MXFP8 for gate/up)
    def _mx_linear(self, idx, Xmx, out=None, residual=None, swiglu_mx=False):
        L = self.layers[idx]
        name = self.LAYER_NAMES[idx]
        T = self.T[: Xmx[0].shape[0]]
        self._mark(f"{name}.down")
        fsd.mx_lora_down(*Xmx, *L["Aq"], self.scale, T)
        self._mark(f"{name}.quant_t")
        fsd.mx_quantize(T, *self.tq)
        self._mark(f"{name}.up")
        if swiglu_mx:
            fsd.mx_lora_up_swiglu_mx(*Xmx, *L["W0q"], *self.tq, *L["Bq"], Hq=self.gq[0],
                                     Hs=self.gq[1])
        else:
            fsd.mx_lora_up(*Xmx, *L["W0q"], *self.tq, *L["Bq"], residual=residual, out=out)

    def _quantize(self, name, X, buf):
        self._mark(name)
        fsd.mx_quantize(X, *buf)
        return buf

    def _blocks(self):
        """embed, then the four linears; leaves the block output in self.h."""
        D = self.D
        self._mark("embed")
        fsd.token_embed(self.z, self.E, out=self.h)
        if self.mx:
            self._mx_linear(0, self._quantize("qkv.quant_x", self.h, self.hq), self.qkv)
            V = self.qkv[:, 2 * D:3 * D]
            self._mx_linear(1, self._quantize("o.quant_x", V, self.vq), self.h, residual=self.h)
            self._mx_linear(2, self._quantize("gate_up.quant_x", self.h, self.hq),
                            swiglu_mx=True)
            self._mx_linear(3, self.gq, self.h, residual=self.h)
        else:
            self._linear(0, self.h, self.qkv)
            self._linear(1, self.qkv[:, 2 * D:3 * D], self.h, residual=self.h)
            self._linear(2, self.h, self.g, epilogue=fsd.EPI_SWIGLU)
            self._linear(3, self.g, self.h, residual=self.h)

    def velocity(self):
        """v = stand-in(z) for the current latent self.z."""
        self._blocks()
        self._mark("head")
        fsd.token_head(self.h, self.P, out=self.v)
        return self.v

    def velocity_euler(self, sigma, sigma_next):
        """The velocity with the Euler update fused into the head: z += (sigma_next - sigma)·v
        without v going through HBM (bitwise equal to velocity() then euler_step)."""
        self._blocks()
        self._mark("head_euler")
        fsd.token_head_euler(self.h, self.P, self.z, sigma, sigma_next)
        return self.z

    def step(self, k, sigmas=SIGMAS, fused=False):
        """Sampler step k: one velocity evaluation and one Euler update, sigmas[k] -> sigmas[k+1]."""
        if fused:
            self.velocity_euler(sigmas[k], sigmas[k + 1])
        else:
            self.velocity()
            self._mark("euler")
            fsd.euler_step(self.z, self.v, sigmas[k], sigmas[k + 1])

    def refine(self, u, eps, sigmas=SIGMAS, fused=False):
        """Renoise u with eps at sigmas[0], then one Euler step per sigma pair."""
        self._mark("renoise")
        fsd.renoise(u, eps, sigmas[0], out=self.z)
        for k in range(len(sigmas) - 1):
            self.step(k, sigmas, fused)
        self._mark("end")
        return self.z

    def capture_steps(self, sigmas=SIGMAS, fused=True):
        """One HIP graph per sampler step (the launches of step k over this refiner's fixed
        buffers, sigmas baked in).  Replaying graph k performs step k on self.z; the renoise
        stays an ordinary launch.  Nothing is allocated inside the captured region."""
        self.events = None
        graphs = []
        side = torch.cuda.Stream(device=self.dev)
        for k in range(len(sigmas) - 1):
            g = torch.cuda.CUDAGraph()
            side.wait_stream(torch.cuda.current_stream(self.dev))
            with torch.cuda.graph(g, stream=side):
                self.step(k, sigmas, fused)
            torch.cuda.current_stream(self.dev).wait_stream(side)
            graphs.append(g)
        return graphs

    def refine_graphs(self, graphs, u, eps, sigmas=SIGMAS):
        """refine() through graphs from capture_steps()."""
        fsd.renoise(u, eps, sigmas[0], out=self.z)
        for g in graphs:
            g.replay()
        return self.z

    def flops_per_step(self) -> dict:
        """Algorithmic flops of one refine (all sigma steps): 2M(KN + Kr + rN) per linear."""
        M, D, F, C, r = self.M, self.D, self.F, self.C, self.R
        steps = len(SIGMAS) - 1
        out = {}
        for L, name in zip(self.layers, self.LAYER_NAMES):
            K, N = L["K"], L["N"]
            out[name + ".down"] = 2 * M * K * r * steps
            out[name + ".up"] = 2 * M * (K + r) * N * steps
        out["embed"] = 2 * M * C * D * steps
        out["head"] = 2 * M * D * C * steps
        return out
