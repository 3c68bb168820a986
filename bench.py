"""Benchmark of the refiner's hot path on one MI355X.

One step = the whole hot path over the 2K grid: renoise a 24-channel
37x90x160 latent (532,800 tokens) at sigma 0.909, then three times
[velocity stand-in = embed, QKV, O(V)+res, gate/up+SwiGLU, down+res, head —
every linear a LoRA-fused linear with the merged rank-576 adapter — then one
Euler update], sigma 0.909 -> 0.857 -> 0.667 -> 0.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value      algorithmic TFLOP/s of the whole step (inputs resident in HBM)
  roofline   the dominant kernel: the gate/up linear's pair launches (phase B
             of a 21,760-token chunk with the SwiGLU epilogue, together with
             phase A of the next chunk): their algorithmic flops per launch /
             their mean launch time from HIP events on their stream, against
             2500 TFLOP/s bf16
  kernels    the same for every kernel of the step
  elementwise  renoise / Euler GB/s at the 768P, 2K and 4K latents, 12 bytes
             per element: batches of back-to-back launches, cache-cold
             (launches cycle through >= 2 GiB of distinct buffers) and warm;
             median / min / max of 5 batches
  graph_fused  the step as one replayed HIP graph per sampler step with the
             Euler update fused into the head
  mxfp8      the step with the four linears as MXFP8 GEMMs (quantization in the
             step time), the fused SwiGLU->MXFP8 gate/up GEMM against the
             5000 TFLOP/s fp8 peak
  lora_linear_configs  the whole LoRA-fused linear at the 768P shape, on one
             4K chunk and over the whole 4K grid chunk by chunk (gate/up with
             SwiGLU chained into down with the residual): median / min / max
             of 20 calls, and the median of 3
  attention_step  the same refine with dense attention between QKV and O
             (all 532,800 tokens as one sequence, 24 heads of 128): step time
             and the attention kernel against 2500 TFLOP/s
  cpu_baseline the fp64 oracle on a bounded sample of tokens on host cores
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (MXFP8 scaled MFMA included)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
DOMINANT = "gate_up.pair"     # phase B of a gate/up chunk + phase A of the next, one launch
SPIN_CYCLES = 200_000          # ~0.1 ms GPU spin queued ahead of a timed region
# ahead of a batch of short launches: long enough (~2 ms) for the host to queue
# the whole batch through the binding before the GPU reaches the first event,
# so the batch runs back to back without waiting on the host
BATCH_SPIN_CYCLES = 4_000_000


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=7)     # 21 launches of each linear kernel
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-elementwise", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target host time of the oracle sample")
    ap.add_argument("--no-mx", action="store_true", help="skip the MXFP8 step")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the refine with dense attention between QKV and O")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the LoRA linears at the 768P and 4K-chunk shapes")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip phase B beside torch.matmul (the BLAS library) at the 2K shapes")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip the step over one GPU's 1/8 share of the tokens")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy first (a known-size kernel for counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_pair_2k_pmc_traffic.md")
GEMM_SOURCE = os.path.join(ROOT, "few_step_diffusion_amd", "csrc", "gemm.hip")


def measured_traffic(kernel):
    """HBM-side bytes per launch of `kernel` (a gemm_kernel template signature)
    from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when
    the GEMM source has changed since those counters were taken."""
    import hashlib
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                key, sep, val = line.strip().partition(": ")
                if sep:
                    fields[key] = val.strip()
        with open(GEMM_SOURCE, "rb") as f:
            cur = hashlib.sha256(f.read()).hexdigest()
        if fields.get("source_sha256") != cur:
            return None
        return int(float(fields["bytes_per_launch " + kernel]))
    except (OSError, KeyError, ValueError):
        return None


def kernel_times(events):
    """Per-name list of durations (ms) between consecutive marks."""
    out = {}
    for (name, a), (_, b) in zip(events[:-1], events[1:]):
        out.setdefault(name, []).append(a.elapsed_time(b))
    return out


def elementwise(torch, fsd, inputs, batches=5, per_batch=24):
    """Renoise / Euler bandwidth at the 768P, 2K and 4K latents.

    Each batch is `per_batch` launches back to back between one pair of HIP
    events, so the figure is the sustained per-launch time, gaps between
    launches included, without a per-launch event overhead (a few us against
    a 25 us kernel at 2K).  cold: consecutive launches cycle through enough
    distinct buffer sets (>= 2 GiB together) that none finds its operands in L2
    or the 256 MB Infinity Cache; warm: every launch reuses one set.  Median,
    min and max of `batches` batches after one untimed batch.
    """
    dev = torch.device("cuda:0")
    res = {}
    for wid, tag in ((1, "768p"), (2, "2k"), (3, "4k")):
        n = inputs.WORKLOADS[wid].latent_elems
        nbytes = 12 * n
        nsets = min(64, max(4, -(-(2 << 30) // nbytes)))
        sets = [(torch.randn(n, device=dev), torch.randn(n, device=dev),
                 torch.empty(n, device=dev)) for _ in range(nsets)]
        for name in ("renoise", "euler"):
            for mode in ("cold", "warm"):
                def launch(k):
                    u, e, z = sets[k % nsets] if mode == "cold" else sets[0]
                    if name == "renoise":
                        fsd.renoise(u, e, 0.909, out=z)
                    else:
                        fsd.euler_step(z, e, 0.909, 0.857)
                ts = []
                for rep in range(batches + 1):
                    torch.cuda._sleep(BATCH_SPIN_CYCLES)
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record()
                    for k in range(per_batch):
                        launch(k)
                    b.record()
                    torch.cuda.synchronize()
                    if rep > 0:
                        ts.append(a.elapsed_time(b) / per_batch)
                med = statistics.median(ts)
                gbs = nbytes / (med * 1e-3) / 1e9
                key = f"{name}_{tag}" if mode == "cold" else f"{name}_{tag}_warm"
                res[key] = {"us": round(med * 1e3, 2), "min_us": round(min(ts) * 1e3, 2),
                            "max_us": round(max(ts) * 1e3, 2), "GB/s": round(gbs, 1),
                            "frac_hbm": round(gbs / PEAK_HBM_GBS, 3), "bytes": nbytes,
                            "buffer_sets": nsets if mode == "cold" else 1}
        del sets
        torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _median_of_3(fn):
    """Median and range of 3 timed runs after one untimed warm-up run."""
    fn()
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        fn()
        runs.append(time.perf_counter() - t0)
    return statistics.median(runs), min(runs), max(runs)


def cpu_baseline(model_flops_per_token, target_s):
    """The fp64 oracle as it stands, timed on the host: median of 3 runs after a
    warm-up, the pages' own method for their timings.
      value          the 2K three-step stand-in (renoise + 3 x (velocity + Euler))
                     on a bounded token sample, algorithmic TFLOP/s of that sample;
      elementwise    renoise + 3 Euler steps with v = eps - x0 on the FULL latent of
                     the 768P, 2K and 4K grids (the oracle's single-threaded loops);
      gemm_rows      the LoRA linear at the 2K QKV and O shapes on a 4,096-row sample
                     (seeded rows of the activations' distribution), with the
                     full-M time extrapolated (rows are independent: cost ~ M)."""
    import numpy as np
    import oracle
    from few_step_diffusion_amd import inputs
    threads = oracle.default_threads()
    out = {"unit": "TFLOP/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
           "host_cpus": os.cpu_count()}
    # --- full-latent sampler (configs 1-3): renoise then 3 Euler steps
    ew = {}
    for wid, tag in ((1, "768p"), (2, "2k"), (3, "4k")):
        u, eps = inputs.latent(wid)
        u, eps = u.numpy().ravel(), eps.numpy().ravel()
        med, lo, hi = _median_of_3(lambda: oracle.sampler_exact_velocity(u, eps))
        n = u.size
        ew[tag] = {"elements": n, "passes": 4, "s_median": round(med, 4),
                   "s_min": round(lo, 4), "s_max": round(hi, 4), "threads": 1,
                   "GB/s_at_12B_per_element_pass": round(4 * 12 * n / med / 1e9, 2)}
        log(f"oracle sampler {tag}: {med:.3f} s")
    out["elementwise"] = ew
    # --- LoRA linear rows at the 2K shapes
    gr = {}
    M2 = inputs.WORKLOADS[2].tokens
    R = 4096
    for layer, (name, K, N, _) in enumerate(inputs.WORKLOADS[2].linears):
        W0 = inputs.base_weight(2, K, N, layer).float().numpy()
        A_l, B_l = inputs.adapters(2, K, N, layer)
        Ab, Bb = oracle.merge_bf16([a.numpy() for a in A_l], [b.numpy() for b in B_l])
        A = oracle.bf16_value(Ab).reshape(Ab.shape)
        B = oracle.bf16_value(Bb).reshape(Bb.shape)
        r = A.shape[0]
        X = inputs.normal((R, K), 1.0, inputs.seed_of(2, inputs.ID_X, 10 + layer))
        X = X.to(__import__("torch").bfloat16).float().numpy()
        oracle.lora_linear_rows(X[:256], W0, A, B, nthreads=threads)      # warm-up
        runs = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.lora_linear_rows(X, W0, A, B, nthreads=threads)
            runs.append(time.perf_counter() - t0)
        med = statistics.median(runs)
        fl = 2.0 * R * (K * N + K * r + r * N)
        gr[name] = {"rows": R, "K": K, "N": N, "r": r, "s_median": round(med, 3),
                    "s_min": round(min(runs), 3), "s_max": round(max(runs), 3),
                    "tflops": round(fl / med / 1e12, 6),
                    "extrapolated_full_s": round(med * M2 / R, 1),
                    "note": f"extrapolated to all {M2:,} rows as t·M/R (not measured)"}
        log(f"oracle LoRA linear {name}: {R} rows {med:.2f} s")
    out["gemm_rows"] = gr
    # --- the stand-in step on a bounded token sample (the value, in the step's unit)
    layers = []
    for L in inputs.standin_layers(4):
        Ab, Bb = oracle.merge_bf16([a.numpy() for a in L["A_list"]],
                                   [b.numpy() for b in L["B_list"]])
        layers.append({"W0": L["W0"].float().numpy(),
                       "A": oracle.bf16_value(Ab).reshape(Ab.shape),
                       "B": oracle.bf16_value(Bb).reshape(Bb.shape)})
    E, P = inputs.standin_projections(4)
    E, P = E.float().numpy(), P.float().numpy()
    u, eps = inputs.latent(4, tokens=4096)
    u, eps = u.numpy(), eps.numpy()
    # warm up and calibrate on one token per thread, then size the sample so
    # that three timed runs take about target_s together; report their median
    t0 = time.perf_counter()
    oracle.standin_refine(u[:threads], eps[:threads], E, P, layers, nthreads=threads)
    t1 = time.perf_counter() - t0
    per_run = target_s / 3
    tokens = int(max(threads, min(4096, threads * max(1.0, per_run / max(t1, 1e-3)))))
    tokens = (tokens // threads) * threads
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.standin_refine(u[:tokens], eps[:tokens], E, P, layers, nthreads=threads)
        runs.append(time.perf_counter() - t0)
    dt = statistics.median(runs)
    out["value"] = round(tokens * model_flops_per_token / dt / 1e12, 6)
    out["extrapolated_full_step_s"] = round(dt * 532800 / tokens, 1)
    out["sample"] = (f"{tokens} of 532,800 tokens of the same step (renoise + 3 stand-in "
                     f"velocity evaluations + Euler), fp64, {threads} threads; median of 3 runs "
                     f"of {min(runs):.1f}-{max(runs):.1f} s after one warm-up; full-step time "
                     "extrapolated (not measured)")
    return out


def attention_step(torch, M, u, eps, args):
    """The refine with dense attention between the QKV and O linears (the pages'
    dense-bf16 baseline refine path): all 532,800 tokens as one sequence, 24
    heads of 128, V's per-head transpose inside each attention call.  One
    untimed refine, then one timed refine with HIP events between launches."""
    from few_step_diffusion_amd.refine import StandinRefiner
    model = StandinRefiner(M, device=u.device, attention=True)
    model.refine(u, eps)
    torch.cuda.synchronize()
    model.events = []
    torch.cuda._sleep(SPIN_CYCLES)
    model.refine(u, eps)
    torch.cuda.synchronize()
    ev = model.events
    model.events = None
    ms = ev[0][1].elapsed_time(ev[-1][1])
    per_kernel = kernel_times(ev)
    flops = model.flops_per_step()
    att = per_kernel["attention"]
    att_ms = statistics.mean(att)
    att_tf = flops["attention"] / len(att) / (att_ms * 1e-3) / 1e12
    tf = sum(flops.values()) / (ms * 1e-3) / 1e12
    log(f"attention step: {ms:.1f} ms, attention {att_ms:.1f} ms per call ({att_tf:.0f} TFLOP/s)")
    del model
    return {"ms_per_step": round(ms, 2), "tflops": round(tf, 1),
            "attention": {"ms_per_call": round(att_ms, 2), "calls_per_step": len(att),
                          "tflops": round(att_tf, 1), "frac_peak": round(att_tf / PEAK_BF16_TFLOPS, 4),
                          "bound": "mfma", "flops_per_call": flops["attention"] / len(att)},
            "tokens": M, "heads": model_heads(), "head_dim": 128,
            "note": "renoise + 3 x (embed, QKV, attention over all 532,800 tokens, O + residual, "
                    "gate/up + SwiGLU, down + residual, head, Euler); attention flops 4·S²·H·D "
                    "per call, including the per-head transpose of V (one pass over V)"}


def model_heads():
    from few_step_diffusion_amd import inputs
    return inputs.STANDIN_D // 128


def mx_step(torch, M, u, eps, flops, bf16_ms, args):
    """The same refine with the four linears as MXFP8 GEMMs, every activation
    quantized by the kernel that produces it (embed, phase A, QKV / O / gate-up
    phase B), inside the step time; per-kernel times and the fused SwiGLU->MXFP8
    gate/up GEMM against the fp8 MFMA peak."""
    from few_step_diffusion_amd.refine import StandinRefiner
    model = StandinRefiner(M, device=u.device, mx=True)
    flops = model.flops_per_step()
    for _ in range(max(1, args.warmup)):
        model.refine(u, eps)
    torch.cuda.synchronize()
    step_events = []
    torch.cuda._sleep(SPIN_CYCLES)
    for _ in range(args.steps):
        model.events = []
        model.refine(u, eps)
        step_events.append(model.events)
    torch.cuda.synchronize()
    model.events = None
    step_ms, per_kernel = [], {}
    for ev in step_events:
        step_ms.append(ev[0][1].elapsed_time(ev[-1][1]))
        for k, v in kernel_times(ev).items():
            per_kernel.setdefault(k, []).extend(v)
    ms = statistics.mean(step_ms)
    total = sum(flops.values())
    kernels = {}
    for name, ts in per_kernel.items():
        ent = {"launches_per_step": len(ts) // args.steps,
               "mean_us": round(statistics.mean(ts) * 1e3, 1),
               "median_us": round(statistics.median(ts) * 1e3, 1)}
        if name in flops:
            per_launch = flops[name] / (len(ts) / args.steps)
            ent["flops_per_launch"] = per_launch
            ent["tflops"] = round(per_launch / (statistics.mean(ts) * 1e-3) / 1e12, 1)
            ent["frac_fp8_peak"] = round(ent["tflops"] / PEAK_FP8_TFLOPS, 4)
        kernels[name] = ent
    lin = [k for k in per_kernel if k.split(".")[0] in StandinRefiner.LAYER_NAMES]
    lin_ms = sum(statistics.mean(per_kernel[k]) * len(per_kernel[k]) / args.steps for k in lin)
    lin_flops = sum(v for k, v in flops.items() if k.split(".")[0] in StandinRefiner.LAYER_NAMES)
    chunked = "gate_up.pair" in kernels          # fsd_mx_lora_linear's pair launches
    dom = kernels["gate_up.pair" if chunked else "gate_up.up"]
    log(f"MXFP8 step {ms:.2f} ms (bf16 {bf16_ms:.2f} ms)")
    del model
    return {"ms_per_step": round(ms, 3), "tflops": round(total / (ms * 1e-3) / 1e12, 1),
            "speedup_vs_bf16": round(bf16_ms / ms, 3),
            "linears": {"ms_per_step": round(lin_ms, 3),
                        "tflops": round(lin_flops / (lin_ms * 1e-3) / 1e12, 1),
                        "note": "phase A writing T as MXFP8, then phase B writing its output "
                                "and the MXFP8 the next linear reads, in the same pass"},
            "dominant": {"kernel": "gate/up phase B, MXFP8 operands, SwiGLU -> MXFP8 epilogue"
                                   + (" (pair launch with phase A of the next chunk)"
                                      if chunked else ""),
                         "bound": "mfma", "achieved": dom["tflops"], "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": dom["frac_fp8_peak"],
                         "flops_per_launch": dom["flops_per_launch"],
                         "traffic": measured_traffic("gemm_pair_mx_kernel<true, true>" if chunked
                                                     else "gemm_kernel<2, 4, true, true, true>")},
            "kernels": kernels,
            "note": "E4M3 elements with E8M0 scales per 32 along K; weights quantized once "
                    "outside the step; flops counted as the bf16 step's (rank 576, K unpadded)"}


def layer_ms_per_call(per_kernel, layer, steps, calls_per_step=3):
    """Mean time of one call of a linear: all of its launches in the timed steps."""
    tot = sum(sum(ts) for k, ts in per_kernel.items() if k.split(".")[0] == layer)
    return tot / (steps * calls_per_step)


def lora_linear_shapes(per_kernel, model, steps):
    """The whole LoRA-fused linear (phase A + phase B, every launch of its
    chunked schedule) at the 2K grid's two shapes, QKV (K = 3072, N = 9216) and
    O (K = N = 3072), from the step's own launches: mean time per call and
    2·M·(K·N + K·r + r·N) flops per call."""
    out = {}
    lf = model.linear_flops()
    for name in ("qkv", "o"):
        ms = layer_ms_per_call(per_kernel, name, steps)
        fl = lf[name]
        tf = fl / (ms * 1e-3) / 1e12
        out[name] = {"ms_per_call": round(ms, 3), "tflops": round(tf, 1),
                     "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4), "flops_per_call": fl,
                     "calls_timed": 3 * steps}
    n, R, _ = __import__("few_step_diffusion_amd").lora_linear_plan(model.M, model.R,
                                                                   model.ws.numel())
    out["note"] = (f"phase A + phase B of one linear over {model.M:,} tokens, rank 576, in "
                   f"{n} launches (chunks of {R} tokens, T in a {model.ws.numel() / 1e6:.1f} MB "
                   "workspace); the O linear's input is the V slice of the QKV output and it "
                   "adds the residual in place")
    return out


def lora_linear_configs(torch, fsd, reps=20, warm=5):
    """The whole LoRA-fused linear (phase A + phase B in one library call) at
    the 768P shape (149,184 tokens, K = N = 3072), on one chunk of the 4K grid
    (299,700 tokens) and over the whole 4K grid (its four chunks in turn):
    gate/up (K = 3072, N = 16384, SwiGLU to 8192) chained into down (K = 8192,
    N = 3072) with the gate/up input as residual.
    Seeded inputs of the workloads' shapes and distributions (activations drawn
    on the device); each call is timed with HIP events on its stream; median,
    min and max over `reps` calls after `warm` warm-up calls, plus the median
    of the first 3 timed calls."""
    from few_step_diffusion_amd import inputs
    dev = torch.device("cuda:0")

    def weights(wid, K, N, layer):
        W0 = inputs.base_weight(wid, K, N, layer).to(dev)
        A_l, B_l = inputs.adapters(wid, K, N, layer)
        A, B = fsd.lora_merge([a.to(dev) for a in A_l], [b.to(dev) for b in B_l])
        return W0, A, B

    def timed(call):
        for _ in range(warm):
            call()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda._sleep(SPIN_CYCLES)
        ev[0].record()
        for i in range(reps):
            call()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]

    def entry(ts, M, K, N, r):
        fl = 2.0 * M * (K * N + K * r + r * N)
        med = statistics.median(ts)
        tf = fl / (med * 1e-3) / 1e12
        return {"tokens": M, "K": K, "N": N, "r": r, "flops_per_call": fl,
                "ms_median": round(med, 3), "ms_min": round(min(ts), 3),
                "ms_max": round(max(ts), 3), "ms_median_of_3": round(statistics.median(ts[:3]), 3),
                "tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                "base_equiv_frac_peak": round(2.0 * M * K * N / (med * 1e-3) / 1e12 /
                                              PEAK_BF16_TFLOPS, 4)}

    out = {}
    wl = inputs.WORKLOADS[1]
    M, (_, K, N, _) = wl.tokens, wl.linears[0]
    W0, A, B = weights(1, K, N, 0)
    X = inputs.activations(1, M, K, device=dev)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(fsd.workspace_bytes(M, A.shape[0]), dtype=torch.uint8, device=dev)
    ts = timed(lambda: fsd.lora_linear(X, W0, A, B, out=Y, workspace=ws))
    out["768p"] = entry(ts, M, K, N, A.shape[0])
    log(f"768P LoRA linear: {out['768p']['ms_median']:.3f} ms, {out['768p']['tflops']} TFLOP/s")
    del W0, A, B, X, Y, ws

    wl = inputs.WORKLOADS[3]
    M = wl.tokens // wl.chunks
    (_, K1, N1, _), (_, K2, N2, _) = wl.linears
    Wg, Ag, Bg = weights(3, K1, N1, 1)
    Wd, Ad, Bd = weights(3, K2, N2, 2)
    Xall = inputs.activations(3, wl.tokens, K1, device=dev)
    X = Xall[:M]
    H = torch.empty((M, N1 // 2), dtype=torch.bfloat16, device=dev)
    Yall = torch.empty((wl.tokens, N2), dtype=torch.bfloat16, device=dev)
    Y = Yall[:M]
    ws = torch.empty(fsd.workspace_bytes(M, Ag.shape[0]), dtype=torch.uint8, device=dev)
    tg = timed(lambda: fsd.lora_linear(X, Wg, Ag, Bg, epilogue="swiglu", out=H, workspace=ws))
    td = timed(lambda: fsd.lora_linear(H, Wd, Ad, Bd, residual=X, out=Y, workspace=ws))
    out["4k_chunk_gate_up"] = entry(tg, M, K1, N1, Ag.shape[0])
    out["4k_chunk_down"] = entry(td, M, K2, N2, Ad.shape[0])
    log(f"4K chunk: gate/up {out['4k_chunk_gate_up']['ms_median']:.3f} ms, "
        f"down {out['4k_chunk_down']['ms_median']:.3f} ms")

    def whole_grid():
        for c in range(wl.chunks):
            rows = slice(c * M, (c + 1) * M)
            fsd.lora_linear(Xall[rows], Wg, Ag, Bg, epilogue="swiglu", out=H, workspace=ws)
            fsd.lora_linear(H, Wd, Ad, Bd, residual=Xall[rows], out=Yall[rows], workspace=ws)
    tw = timed(whole_grid)
    r = Ag.shape[0]
    fl = sum(2.0 * wl.tokens * (K * N + K * r + r * N) for K, N in ((K1, N1), (K2, N2)))
    med = statistics.median(tw)
    out["4k_whole"] = {"tokens": wl.tokens, "chunks": wl.chunks, "flops_per_call": fl,
                       "ms_median": round(med, 3), "ms_min": round(min(tw), 3),
                       "ms_max": round(max(tw), 3),
                       "tflops": round(fl / (med * 1e-3) / 1e12, 1),
                       "frac_peak": round(fl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "note": "all four chunks: gate/up with SwiGLU, then down with the "
                               "gate/up input as residual, per chunk"}
    log(f"4K whole grid ({wl.chunks} chunks): {med:.3f} ms, {out['4k_whole']['tflops']} TFLOP/s")
    out["note"] = ("fsd_lora_linear calls (phase A + phase B); flops 2·M·(K·N + K·r + r·N) with "
                   "r = 576; base_equiv_frac_peak counts 2·M·K·N only")
    del Wg, Ag, Bg, Wd, Ad, Bd, Xall, X, H, Yall, Y, ws
    return out


def vendor_gemm(torch, fsd, reps=10, warm=3):
    """Phase B of the 2K QKV and O linears beside the BLAS library torch calls,
    on the same box in the same run: Y = [X | T]·[W0 | B]ᵀ over 532,800 tokens,
    K = 3072 + 576, N = 9216 and 3072.  Ours is fsd_lora_up in one launch over
    all tokens; the library's is torch.matmul on the K-concatenated operands
    (the same multiply-adds).  Seeded N(0, 1) bf16 operands; each call timed
    with HIP events, median of `reps` after `warm` warm-up calls; the two
    outputs are compared on their first 256 rows."""
    dev = torch.device("cuda:0")
    M, K, r = 532800, 3072, 576
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    Xc = torch.randn((M, K + r), generator=g, device=dev).to(torch.bfloat16)
    X, T = Xc[:, :K], Xc[:, K:]

    def timed(call):
        for _ in range(warm):
            call()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda._sleep(SPIN_CYCLES)
        ev[0].record()
        for i in range(reps):
            call()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return statistics.median(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))

    out = {}
    for name, N in (("qkv", 9216), ("o", 3072)):
        W0 = (torch.randn((N, K), generator=g, device=dev) / K ** 0.5).to(torch.bfloat16)
        B = (torch.randn((N, r), generator=g, device=dev) / r ** 0.5).to(torch.bfloat16)
        Wc = torch.cat([W0, B], dim=1)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        Yv = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ours = timed(lambda: fsd.lora_up(X, W0, T, B, out=Y))
        lib = timed(lambda: torch.matmul(Xc, Wc.t(), out=Yv))
        a, b = Y[:256].float(), Yv[:256].float()
        diff = ((a - b).norm(dim=1) / b.norm(dim=1).clamp_min(1e-30)).max().item()
        fl = 2.0 * M * (K + r) * N
        out[name] = {"N": N, "flops_per_call": fl,
                     "ours_ms": round(ours, 3),
                     "ours_frac_peak": round(fl / (ours * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "library_ms": round(lib, 3),
                     "library_frac_peak": round(fl / (lib * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "max_row_rel_diff_first_256_rows": round(diff, 6)}
        log(f"phase B {name}: ours {ours:.3f} ms, library {lib:.3f} ms")
        del W0, B, Wc, Y, Yv
        torch.cuda.empty_cache()
    out["library"] = str(torch.backends.cuda.preferred_blas_library())
    out["note"] = ("phase B alone, unchunked, one launch over all tokens (no phase A, no T "
                   "production): the library's GEMM does the same multiply-adds")
    return out


def shard_step(torch, M, u, eps, args, shards=8):
    """The bf16 step on one GPU's share of the 2K grid when the tokens are split
    over `shards` GPUs (contiguous token ranges, weights replicated): the kernels
    at the shape each GPU would run.  Nothing is exchanged between shards on
    this path, so this is the per-GPU work of that configuration."""
    from few_step_diffusion_amd.refine import StandinRefiner
    Ms = M // shards
    model = StandinRefiner(Ms, device=u.device)
    us, es = u[:Ms].contiguous(), eps[:Ms].contiguous()
    for _ in range(max(1, args.warmup)):
        model.refine(us, es)
    torch.cuda.synchronize()
    step_events = []
    torch.cuda._sleep(SPIN_CYCLES)
    for _ in range(args.steps):
        model.events = []
        model.refine(us, es)
        step_events.append(model.events)
    torch.cuda.synchronize()
    model.events = None
    step_ms, per_kernel = [], {}
    for ev in step_events:
        step_ms.append(ev[0][1].elapsed_time(ev[-1][1]))
        for k, v in kernel_times(ev).items():
            per_kernel.setdefault(k, []).extend(v)
    flops = model.flops_per_step()
    ms = statistics.mean(step_ms)
    gu_ms = layer_ms_per_call(per_kernel, "gate_up", args.steps)
    dom_tf = model.linear_flops()["gate_up"] / (gu_ms * 1e-3) / 1e12
    log(f"shard of 1/{shards}: {Ms} tokens, {ms:.2f} ms per step")
    del model
    return {"tokens": Ms, "shards": shards, "ms_per_step": round(ms, 3),
            "tflops": round(sum(flops.values()) / (ms * 1e-3) / 1e12, 1),
            "gate_up_linear_tflops": round(dom_tf, 1),
            "gate_up_linear_frac_peak": round(dom_tf / PEAK_BF16_TFLOPS, 4),
            "note": "the same step over one GPU's contiguous 1/8 of the 2K tokens; per-GPU "
                    "figure, no collective on this path (not a measured multi-GPU run)"}


def main():
    args = parse()
    if args.gpus != 1:
        sys.exit("bench.py runs on one GPU only: there is no multi-GPU path (each GPU "
                 "would take a contiguous token range of the latent and exchange nothing)")
    import torch
    import few_step_diffusion_amd as fsd
    from few_step_diffusion_amd import inputs
    from few_step_diffusion_amd.refine import StandinRefiner

    dev = torch.device("cuda:0")
    fsd.lib()
    wl = inputs.WORKLOADS[4]
    M = wl.tokens
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"building the stand-in for {M} tokens ...")
    model = StandinRefiner(M, device=dev)
    u, eps = inputs.latent(4)
    u, eps = u.to(dev), eps.to(dev)
    torch.cuda.synchronize()
    for w in range(args.warmup):
        model.refine(u, eps)
        torch.cuda.synchronize()
        log(f"warmup {w + 1}/{args.warmup} done")
    per_kernel = {}
    step_ms = []
    step_events = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    # the K steps run back to back (events are read after the final sync), so
    # every launch is queued behind running work and each interval between
    # marks is kernel time, not host launch latency
    torch.cuda._sleep(SPIN_CYCLES)
    for s in range(args.steps):
        model.events = []
        model.refine(u, eps)
        step_events.append(model.events)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t_start) / args.steps * 1e3
    for s, ev in enumerate(step_events):
        step_ms.append(ev[0][1].elapsed_time(ev[-1][1]))
        for k, v in kernel_times(ev).items():
            per_kernel.setdefault(k, []).extend(v)
        log(f"step {s + 1}/{args.steps}: {step_ms[-1]:.2f} ms")
    model.events = None

    flops = model.flops_per_step()
    total_flops = sum(flops.values())
    ms = statistics.mean(step_ms)
    value = total_flops / (ms * 1e-3) / 1e12
    steps_per_refine = 3
    kernels = {}
    for name, ts in per_kernel.items():
        mean = statistics.mean(ts)
        ent = {"launches_per_step": len(ts) // args.steps, "mean_us": round(mean * 1e3, 1),
               "median_us": round(statistics.median(ts) * 1e3, 1),
               "min_us": round(min(ts) * 1e3, 1), "max_us": round(max(ts) * 1e3, 1)}
        if name in flops:
            per_launch = flops[name] / (len(ts) / args.steps)
            ent["flops_per_launch"] = per_launch
            ent["tflops"] = round(per_launch / (mean * 1e-3) / 1e12, 1)
            ent["frac_peak"] = round(ent["tflops"] / PEAK_BF16_TFLOPS, 4)
        if name in ("renoise", "euler"):
            ent["GB/s"] = round(12.0 * model.M * model.C / (mean * 1e-3) / 1e9, 1)
        kernels[name] = ent
    lin_names = [k for k in per_kernel if k.split(".")[0] in StandinRefiner.LAYER_NAMES]
    lora_flops = sum(v for k, v in flops.items() if k.split(".")[0] in StandinRefiner.LAYER_NAMES)
    lora_ms = sum(sum(per_kernel[k]) / args.steps for k in lin_names)
    dom = kernels[DOMINANT]
    dom_flops = dom["flops_per_launch"]
    L = model.layers[2]
    _, R, _ = fsd.lora_linear_plan(M, model.R, model.ws.numel())
    traffic = measured_traffic("gemm_pair_kernel<true>")
    roofline = {"kernel": "gate/up linear, one pair launch: phase B (SwiGLU epilogue) of a "
                          f"{R}-token chunk, K={L['K']}+{model.R} N={L['N']}, with phase A "
                          f"(K={L['K']} r={model.R}) of the next chunk",
                "bound": "mfma", "achieved": round(dom_flops / (dom["mean_us"] * 1e-6) / 1e12, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dom_flops / (dom["mean_us"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "flops_per_launch": dom_flops,
                "launches_per_step": dom["launches_per_step"]}
    out = {
        "metric": "LoRA-linear TFLOP/s & % bf16 MFMA peak at 2K grid; renoise/Euler HBM GB/s",
        "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "wall_ms_per_step": round(wall, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "2K three-step sweep: renoise + 3 x (4-layer LoRA stand-in "
                               "d=3072 ffn=8192 r=576=384|128|64 + Euler) over a 24x37x90x160 "
                               "latent", "tokens": M, "global_batch": M, "seq_len": M,
                   "parallelism": "single GPU"},
        "lora_linear": {"tflops": round(lora_flops / (lora_ms * 1e-3) / 1e12, 1),
                        "frac_peak": round(lora_flops / (lora_ms * 1e-3) / 1e12 /
                                           PEAK_BF16_TFLOPS, 4),
                        "ms_per_step": round(lora_ms, 3)},
        "roofline": roofline,
        "lora_linear_2k": lora_linear_shapes(per_kernel, model, args.steps),
        "kernels": kernels,
    }
    # the same step as one HIP graph per sampler step with the Euler update fused
    # into the head (fewer launches, v never written)
    graphs = model.capture_steps(fused=True)
    for _ in range(max(1, args.warmup)):
        model.refine_graphs(graphs, u, eps)
    torch.cuda.synchronize()
    ga = torch.cuda.Event(enable_timing=True)
    gb = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(SPIN_CYCLES)
    ga.record()
    for _ in range(args.steps):
        model.refine_graphs(graphs, u, eps)
    gb.record()
    torch.cuda.synchronize()
    g_ms = ga.elapsed_time(gb) / args.steps
    out["graph_fused"] = {"ms_per_step": round(g_ms, 3),
                          "tflops": round(total_flops / (g_ms * 1e-3) / 1e12, 1),
                          "note": "renoise + one replayed HIP graph per sampler step, "
                                  "head and Euler fused"}
    log(f"graph + fused head/Euler: {g_ms:.2f} ms per step")
    del graphs, model
    torch.cuda.empty_cache()
    if not args.no_configs:
        log("LoRA linears at the 768P and 4K-chunk shapes ...")
        out["lora_linear_configs"] = lora_linear_configs(torch, fsd)
        torch.cuda.empty_cache()
    if not args.no_vendor:
        log("phase B beside the BLAS library ...")
        out["vendor_gemm_2k"] = vendor_gemm(torch, fsd)
        torch.cuda.empty_cache()
    if not args.no_shard:
        log("step on a 1/8 token shard ...")
        out["shard_2k_of_8"] = shard_step(torch, M, u, eps, args)
        torch.cuda.empty_cache()
    if not args.no_mx:
        log("MXFP8 step ...")
        out["mxfp8"] = mx_step(torch, M, u, eps, flops, ms, args)
        torch.cuda.empty_cache()
    if not args.no_attention:
        log("refine with dense attention at the 2K grid ...")
        out["attention_step"] = attention_step(torch, M, u, eps, args)
        torch.cuda.empty_cache()
    if not args.no_elementwise:
        log("elementwise cold-cache timing ...")
        out["elementwise"] = elementwise(torch, fsd, inputs)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(total_flops / M, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
