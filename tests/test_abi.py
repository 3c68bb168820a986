"""The C ABI without a GPU: the library loads, exports every function that
include/fsd.h declares, and rejects invalid arguments with the documented
status before making any HIP call.  Pointers here are plain addresses that
are never dereferenced (validation only looks at their values)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import few_step_diffusion_amd as fsd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsd.h")

OK, EINVAL, EALIGN, EUNSUP, EWS = 0, 1, 2, 3, 4
P = ctypes.c_void_p


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(fsd_\w+)\s*\(", txt, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fsd.library_path()):
        from few_step_diffusion_amd import build
        build.build()
    return fsd.lib()


def test_exports_every_declared_symbol(L):
    names = declared()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", fsd.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fsd_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(L, n) is not None


def test_version_and_status_strings(L):
    assert L.fsd_abi_version() == 1
    assert L.fsd_status_str(0) == b"FSD_OK"
    assert L.fsd_status_str(4) == b"FSD_EWORKSPACE"
    assert L.fsd_status_str(99) == b"FSD_UNKNOWN"
    # two 21,760-row chunks of T at rank 576 (50.1 MB), all rows for small M
    assert L.fsd_lora_linear_workspace_bytes(532800, 576) == 2 * 21760 * 576 * 2
    assert L.fsd_lora_linear_workspace_bytes(43520, 576) == 43520 * 576 * 2
    assert L.fsd_lora_linear_workspace_bytes(1200, 576) == 1200 * 576 * 2
    assert L.fsd_lora_linear_workspace_bytes(0, 576) == 0


def plan(L, M, r, wsb):
    R, sched = ctypes.c_int64(-1), ctypes.c_int(-1)
    n = L.fsd_lora_linear_plan(M, r, wsb, ctypes.byref(R), ctypes.byref(sched))
    return n, R.value, sched.value


def test_lora_linear_plan(L):
    row = 576 * 2
    # the whole of T fits: phase A, phase B
    assert plan(L, 1200, 576, 1200 * row) == (2, 1200, 0)
    assert plan(L, 1200, 576, 10 ** 9) == (2, 1200, 0)
    # the preferred workspace at 2K: pipelined pairs of 85 row tiles
    n, R, sched = plan(L, 532800, 576, L.fsd_lora_linear_workspace_bytes(532800, 576))
    assert (R, sched) == (21760, 1) and n == -(-532800 // 21760) + 1
    # larger workspaces keep the 21,760-row chunk; smaller ones shrink it to 256 multiples
    assert plan(L, 532800, 576, 400 * 10 ** 6)[1:] == (21760, 1)
    assert plan(L, 10000, 576, 2048 * row)[1:] == (1024, 1)
    assert plan(L, 10000, 576, 1100 * row)[1:] == (512, 1)
    assert plan(L, 10000, 576, 512 * row)[1:] == (256, 1)
    # fewer than 512 rows: 256-row chunks, phase A then B each
    n, R, sched = plan(L, 1000, 576, 300 * row)
    assert (n, R, sched) == (8, 256, 2)
    assert plan(L, 0, 576, 0)[0] == 0
    assert plan(L, 100, 0, 0)[0] == 1                      # no LoRA term: one launch
    assert plan(L, -1, 576, 0)[0] == -1


def test_noalloc_rank_limit_without_a_gpu(L):
    # 256 rows of T must fit in the 50,135,040-byte scratch: r <= 97,920; the
    # limit is checked before any HIP call
    rc = L.fsd_lora_linear_noalloc(a(1), 1024, a(2), a(3), a(4), None, None, 0,
                                   ctypes.c_float(1.0), a(5), 1024, 1200, 1024, 1024, 97928, 0,
                                   None)
    assert rc == EUNSUP


def test_graph_entry_points_reject_null(L):
    h = ctypes.c_void_p()
    assert L.fsd_graph_begin(None) == EINVAL          # the default stream cannot be captured
    assert L.fsd_graph_end(None, ctypes.byref(h)) == EINVAL
    assert L.fsd_graph_end(a(1), None) == EINVAL
    assert L.fsd_graph_launch(None, None) == EINVAL
    assert L.fsd_graph_destroy(None) == OK


def test_lora_linear_launch_index(L):
    def launch(idx, M=1200, wsb=1200 * 576 * 2):
        return L.fsd_lora_linear_launch(a(1), 1024, a(2), a(3), a(4), None, None, 0,
                                        ctypes.c_float(1.0), a(5), 1024, M, 1024, 1024, 576, 0,
                                        a(7), wsb, idx, None)
    assert launch(-1) == EINVAL
    assert launch(2) == EINVAL                              # the plan has launches 0 and 1
    assert launch(0, M=0) == OK
    assert launch(1, M=0) == EINVAL


BASE = 0x100000000


def a(i):
    return P(BASE + i * 0x10000000)


def up(L, **kw):
    args = dict(X=a(1), ldx=1024, W0=a(2), T=a(3), ldt=576, B=a(4), bias=None, res=None,
                ldr=0, Y=a(5), ldy=1024, M=1200, N=1024, K=1024, r=576, epi=0)
    args.update(kw)
    return L.fsd_lora_up(args["X"], args["ldx"], args["W0"], args["T"], args["ldt"], args["B"],
                         args["bias"], args["res"], args["ldr"], args["Y"], args["ldy"],
                         args["M"], args["N"], args["K"], args["r"], args["epi"], None)


def test_lora_up_validation(L):
    assert up(L, X=None) == EINVAL
    assert up(L, X=P(BASE + 0x10000008)) == EALIGN
    assert up(L, K=1020, ldx=1020) == EINVAL
    assert up(L, N=1004) == EINVAL
    assert up(L, r=20, ldt=24) == EINVAL
    assert up(L, ldx=1000) == EINVAL                      # ld < K
    assert up(L, epi=7) == EINVAL
    assert up(L, epi=1, N=1032) == EINVAL                 # SwiGLU needs N % 16 == 0
    assert up(L, epi=1, res=a(6), ldr=512) == EUNSUP      # no residual with SwiGLU
    assert up(L, Y=P(BASE + 0x10000000 + 4096)) == EINVAL  # Y overlaps X
    assert up(L, res=P(BASE + 5 * 0x10000000 + 4096), ldr=1024) == EINVAL  # partial overlap
    assert up(L, M=-1) == EINVAL
    assert up(L, M=0) == OK                               # empty: no launch
    assert up(L, M=0, res=a(5), ldr=1024) == OK           # in-place residual is legal
    assert up(L, N=65536, K=32768, ldx=32768, ldy=65536) == EUNSUP   # > 32-bit offsets
    assert up(L, res=a(6), ldr=1 << 22) == EUNSUP          # 256 residual rows span 2 GiB
    assert up(L, M=0, res=a(6), ldr=(1 << 22) - 8) == OK  # just inside


def test_lora_linear_workspace(L):
    def lin(ws, wsb, M=1200, r=576, A=a(3)):
        return L.fsd_lora_linear(a(1), 1024, a(2), A, a(4), None, None, 0, ctypes.c_float(1.0),
                                 a(5), 1024, M, 1024, 1024, r, 0, ws, wsb, None)
    assert lin(None, 0) == EWS
    assert lin(a(7), 256 * 576 * 2 - 2) == EWS
    assert lin(a(7), 256 * 576 * 2, M=0) == OK
    assert lin(None, 0, M=0, r=0, A=None) == OK
    assert lin(P(BASE + 7 * 0x10000000 + 8), 10 ** 9) == EALIGN
    assert lin(P(BASE + 5 * 0x10000000), 10 ** 9) == EINVAL   # workspace == Y
    assert L.fsd_lora_linear(a(1), 1024, a(2), a(3), a(4), None, None, 0,
                             ctypes.c_float(math.nan), a(5), 1024, 16, 1024, 1024, 576, 0,
                             a(7), 10 ** 9, None) == EINVAL


def test_lora_down_validation(L):
    def down(**kw):
        args = dict(X=a(1), ldx=1024, A=a(2), s=1.0, T=a(3), ldt=576, M=100, K=1024, r=576)
        args.update(kw)
        return L.fsd_lora_down(args["X"], args["ldx"], args["A"], ctypes.c_float(args["s"]),
                               args["T"], args["ldt"], args["M"], args["K"], args["r"], None)
    assert down(r=0) == EINVAL
    assert down(T=None) == EINVAL
    assert down(s=math.inf) == EINVAL
    assert down(T=P(BASE + 3 * 0x10000000 + 2)) == EALIGN
    assert down(T=P(BASE + 0x10000000 + 64)) == EINVAL    # T overlaps X
    assert down(M=0) == OK


def test_sampler_validation(L):
    f = ctypes.c_float
    assert L.fsd_renoise(a(1), a(2), f(0.909), a(3), 0, None) == OK
    assert L.fsd_renoise(a(1), a(2), f(math.nan), a(3), 10, None) == EINVAL
    assert L.fsd_renoise(a(1), a(2), f(0.5), P(BASE + 3 * 0x10000000 + 4), 10, None) == EALIGN
    assert L.fsd_renoise(a(1), a(2), f(0.5), P(BASE + 0x10000000 + 16), 100, None) == EINVAL
    assert L.fsd_renoise(None, a(2), f(0.5), a(3), 10, None) == EINVAL
    assert L.fsd_renoise(a(1), a(2), f(0.5), a(3), -1, None) == EINVAL
    assert L.fsd_euler_step(a(1), a(2), f(0.909), f(math.inf), 10, None) == EINVAL
    assert L.fsd_euler_step(a(1), P(BASE + 0x10000000 + 16), f(0.9), f(0.8), 100, None) == EINVAL
    assert L.fsd_euler_step(a(1), a(2), f(0.9), f(0.8), 0, None) == OK


def test_standin_and_merge_validation(L):
    assert L.fsd_token_embed(a(1), a(2), a(3), 3072, 10, 33, 3072, None) == EINVAL
    assert L.fsd_token_embed(a(1), a(2), a(3), 3070, 10, 24, 3072, None) == EINVAL
    assert L.fsd_token_embed(a(1), a(2), a(3), 3072, 0, 24, 3072, None) == OK
    assert L.fsd_token_head(a(1), 3072, a(2), a(3), 10, 3000, 24, None) == EINVAL
    assert L.fsd_token_head(a(1), 3072, a(2), P(BASE + 3 * 0x10000000 + 2), 10, 3072, 24,
                            None) == EALIGN
    f = ctypes.c_float
    assert L.fsd_token_head_euler(a(1), 3072, a(2), a(3), 10, 3072, 24, f(math.nan), f(0.8),
                                  None) == EINVAL
    assert L.fsd_token_head_euler(a(1), 3072, a(2), a(3), 10, 3072, 33, f(0.9), f(0.8),
                                  None) == EINVAL
    assert L.fsd_token_head_euler(a(1), 3072, a(2), P(BASE + 3 * 0x10000000 + 2), 10, 3072, 24,
                                  f(0.9), f(0.8), None) == EALIGN
    assert L.fsd_token_head_euler(a(1), 3072, a(2), P(BASE + 0x10000000 + 64), 10, 3072, 24,
                                  f(0.9), f(0.8), None) == EINVAL        # z overlaps H
    assert L.fsd_token_head_euler(a(1), 3072, a(2), a(3), 0, 3072, 24, f(0.9), f(0.8),
                                  None) == OK
    arr = (P * 1)(a(1))
    rk = (ctypes.c_int64 * 1)(8)
    assert L.fsd_lora_merge(0, arr, arr, rk, None, 16, 16, a(2), a(3), None) == EINVAL
    assert L.fsd_lora_merge(1, arr, arr, rk, None, 16, 16, P(BASE + 2 * 0x10000000 + 8), a(3),
                            None) == EALIGN
    assert L.fsd_lora_merge(1, arr, arr, rk, None, 16, 16, a(2), a(2), None) == EINVAL


def test_mx_validation(L):
    f = ctypes.c_float
    assert L.fsd_mx_scale_bytes(300, 576) == 5 * 512 * 4
    assert L.fsd_mx_scale_bytes(0, 576) == 0
    # quantize
    assert L.fsd_mx_quantize(a(1), 576, 0, 576, a(2), 640, a(3), None) == OK
    assert L.fsd_mx_quantize(a(1), 576, 300, 560, a(2), 640, a(3), None) == EINVAL  # K % 32
    assert L.fsd_mx_quantize(a(1), 576, 300, 576, a(2), 576, a(3), None) == EINVAL  # ldq < Kp
    assert L.fsd_mx_quantize(a(1), 576, 300, 576, a(2), 640, P(BASE + 3 * 0x10000000 + 2),
                             None) == EALIGN                                      # S word-aligned
    assert L.fsd_mx_quantize(a(1), 576, 300, 576, a(2), 640, P(BASE + 0x10000000 + 64),
                             None) == EINVAL                                      # S overlaps X

    def down(**kw):
        args = dict(Xq=a(1), ldxq=1024, Xs=a(2), Aq=a(3), As=a(4), s=1.0, T=a(5), ldt=576,
                    M=100, K=1024, r=576)
        args.update(kw)
        return L.fsd_mx_lora_down(args["Xq"], args["ldxq"], args["Xs"], args["Aq"], args["As"],
                                  f(args["s"]), args["T"], args["ldt"], args["M"], args["K"],
                                  args["r"], None)
    assert down(M=0) == OK
    assert down(K=1000) == EINVAL                        # K % 32
    assert down(ldxq=1000, K=992) == EINVAL              # ldxq < Kp (1024)
    assert down(ldxq=1032) == EINVAL                     # ldxq % 16
    assert down(Xs=None) == EINVAL
    assert down(As=P(BASE + 4 * 0x10000000 + 2)) == EALIGN
    assert down(Aq=P(BASE + 3 * 0x10000000 + 8)) == EALIGN
    assert down(s=math.nan) == EINVAL
    assert down(T=P(BASE + 2 * 0x10000000 + 64)) == EINVAL   # T overlaps Xs
    assert down(r=576, K=4 * 1024 * 1024, ldxq=4 * 1024 * 1024) == EUNSUP

    def upm(**kw):
        args = dict(Xq=a(1), ldxq=1024, Xs=a(2), Wq=a(3), Ws=a(4), Tq=a(5), ldtq=640, Ts=a(6),
                    Bq=a(7), Bs=a(8), bias=None, res=None, ldr=0, Y=a(9), ldy=1024, M=300,
                    N=1024, K=1024, r=576, epi=0)
        args.update(kw)
        return L.fsd_mx_lora_up(args["Xq"], args["ldxq"], args["Xs"], args["Wq"], args["Ws"],
                                args["Tq"], args["ldtq"], args["Ts"], args["Bq"], args["Bs"],
                                args["bias"], args["res"], args["ldr"], args["Y"], args["ldy"],
                                args["M"], args["N"], args["K"], args["r"], args["epi"], None)
    assert upm(M=0) == OK
    assert upm(r=0, Tq=None, Ts=None, Bq=None, Bs=None, M=0) == OK
    assert upm(r=40) == EINVAL                           # r % 32
    assert upm(ldtq=576) == EINVAL                       # ldtq < rp (640)
    assert upm(Ts=None) == EINVAL
    assert upm(Bs=P(BASE + 8 * 0x10000000 + 1)) == EALIGN
    assert upm(epi=1, N=1040) == EUNSUP                  # MX SwiGLU needs N % 128 == 0
    assert upm(epi=1, N=1032) == EINVAL                  # ... and N % 16 as always
    assert upm(epi=1, res=a(10), ldr=512) == EUNSUP
    assert upm(epi=3) == EINVAL
    assert upm(Y=P(BASE + 7 * 0x10000000 + 4096)) == EINVAL   # Y overlaps Bq
    assert upm(M=0, res=a(9), ldr=1024) == OK            # in-place residual is legal
    assert upm(res=a(10), ldr=1 << 22) == EUNSUP         # 256 residual rows span 2 GiB

    def upq(**kw):
        args = dict(Xq=a(1), ldxq=1024, Xs=a(2), Wq=a(3), Ws=a(4), Tq=a(5), ldtq=640, Ts=a(6),
                    Bq=a(7), Bs=a(8), bias=None, Hq=a(9), ldhq=512, Hs=a(10), M=300, N=1024,
                    K=1024, r=576)
        args.update(kw)
        return L.fsd_mx_lora_up_swiglu_mx(args["Xq"], args["ldxq"], args["Xs"], args["Wq"],
                                          args["Ws"], args["Tq"], args["ldtq"], args["Ts"],
                                          args["Bq"], args["Bs"], args["bias"], args["Hq"],
                                          args["ldhq"], args["Hs"], args["M"], args["N"],
                                          args["K"], args["r"], None)
    assert upq(M=0) == OK
    assert upq(N=1152) == EUNSUP                         # fused quantizer: N % 256 == 0
    assert upq(N=1032) == EINVAL
    assert upq(ldhq=500) == EINVAL                       # ldhq < N/2
    assert upq(ldhq=520) == EINVAL                       # ldhq % 16
    assert upq(Hs=None) == EINVAL
    assert upq(Hs=P(BASE + 10 * 0x10000000 + 2)) == EALIGN
    assert upq(Hq=P(BASE + 9 * 0x10000000 + 8)) == EALIGN
    assert upq(Hs=P(BASE + 9 * 0x10000000 + 4096)) == EINVAL   # Hs overlaps Hq
    assert upq(Hq=P(BASE + 0x10000000 + 4096)) == EINVAL       # Hq overlaps Xq
    assert upq(Hs=P(BASE + 4 * 0x10000000 + 64)) == EINVAL     # Hs overlaps W0s
    assert upq(r=40) == EINVAL


def test_mx_scale_layout_helpers():
    """The host pack / unpack helpers follow the documented layout: byte i of word
    16·b + r of (step t, group g) is row 64g + 16i + r, block 4t + b."""
    import numpy as np
    M, K = 300, 576
    off = fsd.mx_scale_offsets(M, K)
    Mp = 512
    assert off.shape == (M, 20)
    for m, blk in [(0, 0), (17, 1), (63, 3), (64, 4), (299, 19), (130, 9)]:
        t, b = blk // 4, blk % 4
        g, i, r = m // 64, (m % 64) // 16, m % 16
        assert off[m, blk] == ((t * (Mp // 64) + g) * 64 + 16 * b + r) * 4 + i
    assert len(set(off.ravel().tolist())) == off.size   # one byte per scale
    s = np.random.default_rng(0).integers(0, 255, size=(M, 20), dtype=np.uint8)
    S = fsd.mx_pack_scales(s, K)
    assert S.numel() == fsd.mx_scale_bytes(M, K)
    assert np.array_equal(fsd.mx_unpack_scales(S, M, K), s)
    assert int((S.numpy() == 127).sum()) >= (Mp - M) * 20   # padding rows


def test_attention_validation(L):
    f = ctypes.c_float

    def att(**kw):
        args = dict(Q=a(1), K=a(2), V=a(3), ld=9216, O=a(4), ldo=3072, S=1000, H=24, D=128,
                    scale=0.0883883, ws=a(5), wsb=10 ** 9)
        args.update(kw)
        return L.fsd_attention(args["Q"], args["K"], args["V"], args["ld"], args["O"], args["ldo"],
                               args["S"], args["H"], args["D"], f(args["scale"]), args["ws"],
                               args["wsb"], None)
    assert L.fsd_attention_workspace_bytes(1000, 24, 128) == 24 * 128 * 1024 * 2
    assert L.fsd_attention_workspace_bytes(0, 24, 128) == 0
    assert att(S=0) == OK
    assert att(D=64, ldo=1536) == EUNSUP                  # head dim 128 only
    assert att(scale=0.0) == EINVAL
    assert att(scale=math.nan) == EINVAL
    assert att(ld=3000) == EINVAL                         # ld < H·D
    assert att(ldo=3076) == EINVAL                        # ldo % 8
    assert att(ws=None, wsb=0) == EWS
    assert att(wsb=24 * 128 * 1024 * 2 - 2) == EWS
    assert att(O=P(BASE + 4 * 0x10000000 + 8)) == EALIGN
    assert att(ws=P(BASE + 5 * 0x10000000 + 4)) == EALIGN
    assert att(O=P(BASE + 0x10000000 + 4096)) == EINVAL   # O overlaps Q
    assert att(ws=P(BASE + 3 * 0x10000000 + 4096)) == EINVAL   # workspace overlaps V
    assert att(H=0) == EINVAL


def test_python_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        fsd.renoise(torch.zeros(8), torch.zeros(8), 0.5)


def test_one_pass_mx_validation(L):
    f = ctypes.c_float

    def dmx(**kw):
        args = dict(Xq=a(1), ldxq=1024, Xs=a(2), Aq=a(3), As=a(4), s=1.0, Tq=a(5), ldtq=640,
                    Ts=a(6), M=300, K=1024, r=576)
        args.update(kw)
        return L.fsd_mx_lora_down_mx(args["Xq"], args["ldxq"], args["Xs"], args["Aq"],
                                     args["As"], f(args["s"]), args["Tq"], args["ldtq"],
                                     args["Ts"], args["M"], args["K"], args["r"], None)
    assert dmx(M=0) == OK
    assert dmx(r=72) == EINVAL                           # T's blocks: r % 32
    assert dmx(ldtq=576) == EINVAL                       # ldtq < rp (640)
    assert dmx(ldtq=648) == EINVAL                       # ldtq % 16
    assert dmx(Ts=None) == EINVAL
    assert dmx(Ts=P(BASE + 6 * 0x10000000 + 2)) == EALIGN
    assert dmx(s=math.inf) == EINVAL
    assert dmx(Tq=P(BASE + 0x10000000 + 64)) == EINVAL   # Tq overlaps Xq
    assert dmx(Ts=P(BASE + 5 * 0x10000000 + 64)) == EINVAL   # Ts overlaps Tq

    def uq(**kw):
        args = dict(Xq=a(1), ldxq=1024, Xs=a(2), Wq=a(3), Ws=a(4), Tq=a(5), ldtq=640, Ts=a(6),
                    Bq=a(7), Bs=a(8), bias=None, res=None, ldr=0, Y=a(9), ldy=1024, M=300,
                    N=1024, K=1024, r=576, q0=0, q1=1024, Yq=a(10), ldyq=1024, Ys=a(11))
        args.update(kw)
        return L.fsd_mx_lora_up_q(*(args[k] for k in (
            "Xq", "ldxq", "Xs", "Wq", "Ws", "Tq", "ldtq", "Ts", "Bq", "Bs", "bias", "res", "ldr",
            "Y", "ldy", "M", "N", "K", "r", "q0", "q1", "Yq", "ldyq", "Ys")), None)
    assert uq(M=0) == OK
    assert uq(M=0, res=a(9), ldr=1024) == OK             # in-place residual is legal
    assert uq(q0=16) == EINVAL                           # q0 % 32
    assert uq(q1=1000) == EINVAL                         # q1 % 32
    assert uq(q0=512, q1=512) == EINVAL                  # empty range
    assert uq(q1=1056) == EINVAL                         # past N
    assert uq(q0=-32) == EINVAL
    assert uq(q0=32, q1=352, ldyq=320) == EINVAL         # ldyq < 384 (320 padded to 128)
    assert uq(q0=32, q1=352, ldyq=384, M=0) == OK
    assert uq(Y=None) == EINVAL
    assert uq(Ys=None) == EINVAL
    assert uq(Yq=P(BASE + 10 * 0x10000000 + 8)) == EALIGN
    assert uq(Yq=P(BASE + 9 * 0x10000000 + 4096)) == EINVAL    # Yq overlaps Y
    assert uq(Ys=P(BASE + 10 * 0x10000000 + 4096)) == EINVAL   # Ys overlaps Yq
    assert uq(Ys=P(BASE + 7 * 0x10000000 + 64)) == EINVAL      # Ys overlaps Bq
    assert uq(res=a(12), ldr=1024, Yq=P(BASE + 12 * 0x10000000 + 64)) == EINVAL  # Yq over res

    def emx(**kw):
        args = dict(z=a(1), E=a(2), X=a(3), ldx=3072, M=100, C=24, D=3072, Xq=a(4), ldxq=3072,
                    Xs=a(5))
        args.update(kw)
        return L.fsd_token_embed_mx(*(args[k] for k in (
            "z", "E", "X", "ldx", "M", "C", "D", "Xq", "ldxq", "Xs")), None)
    assert emx(M=0) == OK
    assert emx(D=3008, ldx=3008, ldxq=3008) == EUNSUP    # D % 128
    assert emx(C=33) == EINVAL
    assert emx(ldxq=3056) == EINVAL                      # ldxq < D
    assert emx(Xs=None) == EINVAL
    assert emx(Xq=P(BASE + 4 * 0x10000000 + 4)) == EALIGN
    assert emx(Xq=P(BASE + 3 * 0x10000000 + 4096)) == EINVAL   # Xq overlaps X
    assert emx(Xs=P(BASE + 0x10000000 + 16)) == EINVAL         # Xs overlaps z


def test_mx_lora_linear_plan_and_validation(L):
    f = ctypes.c_float
    rp_row = 640 + 20                                  # codes + scales per row of T, r = 576
    assert L.fsd_mx_lora_linear_workspace_bytes(532800, 576) == 2 * 21760 * rp_row
    assert L.fsd_mx_lora_linear_workspace_bytes(1000, 576) == 2 * 1024 * rp_row
    assert L.fsd_mx_lora_linear_workspace_bytes(0, 576) == 0
    n, R = ctypes.c_int64(), ctypes.c_int64()

    def plan(M, r, ws):
        st = L.fsd_mx_lora_linear_plan(M, r, ws, ctypes.byref(n), ctypes.byref(R))
        return st, n.value, R.value
    assert plan(532800, 576, 2 * 21760 * rp_row) == (OK, -(-532800 // 21760) + 1, 21760)
    assert plan(532800, 576, 10 ** 9)[2] == 21760          # capped at 85 row tiles
    assert plan(5037, 576, 2 * 256 * rp_row) == (OK, 21, 256)
    assert plan(5037, 576, 2 * 256 * rp_row - 1)[0] == EWS   # not two 256-row chunks
    assert plan(1, 64, 2 * 256 * (128 + 4))[1:] == (2, 256)
    assert plan(100, 40, 10 ** 6)[0] == EINVAL               # r % 32
    # at a huge rank the chunk's T scales (R·rp/32 bytes) must stay below 2^31
    big_r = 1 << 22
    cap = (0x7FFFFFFF // (big_r // 32)) // 256 * 256
    assert cap < 21760
    assert L.fsd_mx_lora_linear_workspace_bytes(10 ** 6, big_r) == 2 * cap * (big_r + big_r // 32)
    assert plan(10 ** 6, big_r, 10 ** 12)[2] == cap
    assert L.fsd_mx_lora_linear_plan(100, 64, 10 ** 6, None, ctypes.byref(R)) == EINVAL

    def lin(**kw):
        args = dict(Xq=a(1), ldxq=1024, Xs=a(2), Aq=a(3), As=a(4), s=1.0, Wq=a(5), Ws=a(6),
                    Bq=a(7), Bs=a(8), bias=None, res=None, ldr=0, Y=a(9), ldy=1024, M=300,
                    N=1024, K=1024, r=576, epi=0, q0=0, q1=0, Yq=None, ldyq=0, Ys=None,
                    ws=a(10), wsb=2 * 256 * rp_row)
        args.update(kw)
        return L.fsd_mx_lora_linear(
            args["Xq"], args["ldxq"], args["Xs"], args["Aq"], args["As"], f(args["s"]),
            args["Wq"], args["Ws"], args["Bq"], args["Bs"], args["bias"], args["res"],
            args["ldr"], args["Y"], args["ldy"], args["M"], args["N"], args["K"], args["r"],
            args["epi"], args["q0"], args["q1"], args["Yq"], args["ldyq"], args["Ys"],
            args["ws"], args["wsb"], None)
    assert lin(M=0) == OK
    assert lin(M=0, ws=None, wsb=0) == OK
    assert lin(M=0, res=a(9), ldr=1024) == OK                 # in-place residual
    assert lin(wsb=2 * 256 * rp_row - 1) == EWS
    assert lin(ws=None) == EWS
    assert lin(ws=P(BASE + 10 * 0x10000000 + 8)) == EALIGN
    assert lin(ws=P(BASE + 9 * 0x10000000 + 64)) == EINVAL      # workspace overlaps Y
    assert lin(r=40) == EINVAL
    assert lin(Y=None) == EINVAL                               # plain epilogue needs Y
    assert lin(epi=1, Yq=a(11), Ys=a(12), ldyq=512, q0=0, q1=512) == EINVAL   # SwiGLU: Y xor Yq
    assert lin(M=0, epi=1, Y=None, Yq=a(11), Ys=a(12), ldyq=512, q0=0, q1=512) == OK
    assert lin(epi=1, Y=None, Yq=a(11), Ys=a(12), ldyq=512, q0=0, q1=256) == EINVAL
    assert lin(epi=1, N=1152, Y=None, Yq=a(11), Ys=a(12), ldyq=576, q0=0, q1=576) == EUNSUP
    assert lin(epi=1, res=a(13), ldr=512, ldy=512) == EINVAL   # no residual with SwiGLU
    assert lin(Yq=a(11), Ys=a(12), ldyq=1024, q0=16, q1=1024) == EINVAL
    assert lin(Yq=a(11), Ys=a(12), ldyq=1000, q0=0, q1=1024) == EINVAL
    assert lin(Yq=P(BASE + 9 * 0x10000000 + 4096), Ys=a(12), ldyq=1024, q0=0, q1=1024) == EINVAL
    assert lin(M=0, Yq=a(11), Ys=a(12), ldyq=1024, q0=0, q1=1024) == OK
