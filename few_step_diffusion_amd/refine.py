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

with every L_* the LoRA-fused linear.  With attention=True the O linear reads
dense attention over all tokens instead of the V slice (the pages' baseline
refine runs dense bf16 attention between them; "Where the 3.9x speedup comes
from", dense-BF16 row): h = x + L_o(attention(Q, K, V)), heads of 128.  Every
call below runs HIP kernels of libfsd.so (through the ctypes binding); torch
only allocates device memory and supplies the stream.
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
                 scale: float = 1.0, mx: bool = False, attention: bool = False,
                 mx_onepass: bool = True, mx_chunked: bool = False):
        """mx: run the four linears as MXFP8 GEMMs.  The bf16 weights are quantized
        once here.  Every linear's input and its LoRA down output are the MXFP8 of
        their bf16 values.  mx_onepass (default): each producer writes that MXFP8
        form in the same pass (embed -> QKV input, phase A -> T, QKV phase B -> the
        V slice, O phase B -> the gate/up input, gate/up phase B -> SwiGLU's
        output); otherwise separate quantizer passes read the bf16 values back
        (SwiGLU's output stays fused).  mx_chunked: run each one-pass linear through
        fsd_mx_lora_linear (row chunks, T as MXFP8 in a 28.7 MB workspace) instead of
        phase A over all rows then phase B.  All routes write the same bytes."""
        dev = torch.device(device)
        if attention and (mx or D % 128):
            raise ValueError("the attention step runs on the bf16 path with heads of 128")
        self.M, self.D, self.F, self.C, self.dev = M, D, F, C, dev
        self.attention = attention
        self.heads = D // 128
        self.R = sum(ranks)
        self.scale = scale
        self.mx = mx
        self.onepass = mx and mx_onepass
        self.chunked = self.onepass and mx_chunked
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
        if mx:
            if not self.onepass:
                self.T = torch.empty((M, self.R), dtype=bf, device=dev)  # LoRA down output
        else:
            # T of the bf16 linears: two chunks of 21,760 rows (50 MB at rank 576),
            # shared by the four linears (they run one after another on one stream)
            self.ws = torch.empty(max(fsd.workspace_bytes(M, self.R), 16), dtype=torch.uint8,
                                  device=dev)
        if attention:
            self.att = torch.empty((M, D), dtype=bf, device=dev)      # attention output
            self.att_ws = torch.empty(max(fsd.attention_workspace_bytes(M, self.heads), 16),
                                      dtype=torch.uint8, device=dev)
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
            if self.chunked:
                # T as MXFP8, two chunks of 21,760 rows (28.7 MB at rank 576), shared by
                # the four linears
                self.mx_ws = torch.empty(max(fsd.mx_workspace_bytes(M, self.R), 16),
                                         dtype=u8, device=dev)
            else:
                self.tq = mxbuf(self.R)  # LoRA down output, all rows
            del self.g
        self.events = None

    def launch_names(self):
        """Mark name of each launch of one LoRA linear over this refiner's tokens:
        phase A then phase B ('down', 'up'), or, chunked, phase A of the first
        chunk ('down0') followed by phase-B / next-phase-A pairs ('pair')."""
        if self.chunked:
            n, _ = fsd.mx_lora_linear_plan(self.M, self.R, self.mx_ws.numel())
            return ["down0"] + ["pair"] * (n - 1)
        n, _, sched = fsd.lora_linear_plan(self.M, self.R, self.ws.numel())
        if sched == 1:
            return ["down0"] + ["pair"] * (n - 1)
        return ["down", "up"] * (n // 2)

    # one LoRA linear = phase A + phase B through the chunked schedule
    def _linear(self, idx, X, out, residual=None, epilogue=fsd.EPI_NONE):
        L = self.layers[idx]
        hook = None
        if self.events is not None:
            names = self.launch_names()
            hook = lambda i: self._mark(f"{self.LAYER_NAMES[idx]}.{names[i]}")
        fsd.lora_linear(X, L["W0"], L["A"], L["B"], self.scale, residual=residual,
                        epilogue=epilogue, out=out, workspace=self.ws, on_launch=hook)

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

    # one MXFP8 LoRA linear in row chunks (fsd_mx_lora_linear): T exists only as the
    # MXFP8 of one chunk in the workspace; phase B optionally writes the MXFP8 form
    # of (some of) its output columns, or SwiGLU's output as MXFP8 only
    def _mx_linear_onepass(self, idx, Xmx, out=None, residual=None, swiglu_mx=False,
                           qout=None, cols=None):
        L = self.layers[idx]
        name = self.LAYER_NAMES[idx]
        if not self.chunked:
            # phase A over all rows writing T as MXFP8, then phase B
            self._mark(f"{name}.down")
            fsd.mx_lora_down_mx(*Xmx, *L["Aq"], self.scale, *self.tq)
            self._mark(f"{name}.up")
            if swiglu_mx:
                fsd.mx_lora_up_swiglu_mx(*Xmx, *L["W0q"], *self.tq, *L["Bq"], Hq=self.gq[0],
                                         Hs=self.gq[1])
            elif qout is not None:
                fsd.mx_lora_up_q(*Xmx, *L["W0q"], *self.tq, *L["Bq"], residual=residual,
                                 out=out, cols=cols, Yq=qout[0], Ys=qout[1])
            else:
                fsd.mx_lora_up(*Xmx, *L["W0q"], *self.tq, *L["Bq"], residual=residual, out=out)
            return
        hook = None
        if self.events is not None:
            names = self.launch_names()
            hook = lambda i: self._mark(f"{name}.{names[i]}")
        if swiglu_mx:
            fsd.mx_lora_linear(*Xmx, *L["Aq"], *L["W0q"], *L["Bq"], self.scale,
                               epilogue=fsd.EPI_SWIGLU, Yq=self.gq[0], Ys=self.gq[1],
                               workspace=self.mx_ws, on_launch=hook)
        else:
            fsd.mx_lora_linear(*Xmx, *L["Aq"], *L["W0q"], *L["Bq"], self.scale,
                               residual=residual, out=out, cols=cols,
                               Yq=None if qout is None else qout[0],
                               Ys=None if qout is None else qout[1],
                               workspace=self.mx_ws, on_launch=hook)

    def _quantize(self, name, X, buf):
        self._mark(name)
        fsd.mx_quantize(X, *buf)
        return buf

    def _blocks(self):
        """embed, then the four linears; leaves the block output in self.h."""
        D = self.D
        self._mark("embed")
        if self.onepass:
            fsd.token_embed_mx(self.z, self.E, out=self.h, Xq=self.hq[0], Xs=self.hq[1])
            self._mx_linear_onepass(0, self.hq, self.qkv, qout=self.vq, cols=(2 * D, 3 * D))
            self._mx_linear_onepass(1, self.vq, self.h, residual=self.h, qout=self.hq)
            self._mx_linear_onepass(2, self.hq, swiglu_mx=True)
            self._mx_linear_onepass(3, self.gq, self.h, residual=self.h)
            return
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
            if self.attention:
                self._mark("attention")
                fsd.attention(self.qkv[:, :D], self.qkv[:, D:2 * D], self.qkv[:, 2 * D:3 * D],
                              self.heads, out=self.att, workspace=self.att_ws)
                self._linear(1, self.att, self.h, residual=self.h)
            else:
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
        buffers, sigmas baked in), captured by the library (fsd_graph_begin / _end).
        Replaying graph k performs step k on self.z; the renoise stays an ordinary
        launch.  Nothing is allocated inside the captured region."""
        self.events = None
        graphs = []
        side = torch.cuda.Stream(device=self.dev)
        for k in range(len(sigmas) - 1):
            side.wait_stream(torch.cuda.current_stream(self.dev))
            with fsd.StepGraph.capture(side) as g:
                self.step(k, sigmas, fused)
            torch.cuda.current_stream(self.dev).wait_stream(side)
            graphs.append(g)
        return graphs

    def refine_graphs(self, graphs, u, eps, sigmas=SIGMAS):
        """refine() through graphs from capture_steps()."""
        fsd.renoise(u, eps, sigmas[0], out=self.z)
        for g in graphs:
            g.launch()
        return self.z

    def flops_per_step(self) -> dict:
        """Algorithmic flops of one refine (all sigma steps) per launch mark name:
        2M(KN + Kr + rN) per linear, split over its launches (phase A of a chunk
        2·Mc·K·r, phase B 2·Mc·(K + r)·N), plus embed and head."""
        M, D, F, C, r = self.M, self.D, self.F, self.C, self.R
        steps = len(SIGMAS) - 1
        out = {}
        for L, name in zip(self.layers, self.LAYER_NAMES):
            K, N = L["K"], L["N"]
            down, up = 2 * M * K * r, 2 * M * (K + r) * N
            if self.chunked:
                _, R = fsd.mx_lora_linear_plan(M, r, self.mx_ws.numel())
                first = 2 * min(M, R) * K * r
                out[name + ".down0"] = first * steps
                out[name + ".pair"] = (down - first + up) * steps
                continue
            if self.mx:
                out[name + ".down"] = down * steps
                out[name + ".up"] = up * steps
                continue
            n, R, sched = fsd.lora_linear_plan(M, r, self.ws.numel())
            if sched == 1:
                first = 2 * min(M, R) * K * r
                out[name + ".down0"] = first * steps
                out[name + ".pair"] = (down - first + up) * steps
            else:
                out[name + ".down"] = down * steps
                out[name + ".up"] = up * steps
        out["embed"] = 2 * M * C * D * steps
        out["head"] = 2 * M * D * C * steps
        if self.attention:
            out["attention"] = 4 * M * M * D * steps          # Q·Kᵀ and P·V, all heads
        return out

    def linear_flops(self) -> dict:
        """Algorithmic flops of one call of each linear, 2M(KN + Kr + rN)."""
        return {name: 2 * self.M * (L["K"] * L["N"] + L["K"] * self.R + self.R * L["N"])
                for L, name in zip(self.layers, self.LAYER_NAMES)}
