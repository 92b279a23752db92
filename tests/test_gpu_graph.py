"""The hot path under HIP graph capture: split + compensated GEMM + INT16 quantisation + decode attention
captured once with torch.cuda.graph, then replayed several times with eager work and synchronisations in
between; every replay must equal the eager results bit for bit (the kernels issue no memsets and allocate
nothing of their own; the decode workspace comes from the caller)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import banner, dev

pytestmark = pytest.mark.gpu


def test_hot_path_graph_replays_equal_eager(heal):
    banner("graph capture: split + gemm + quant + decode, 4 replays")
    M, K, N = 96, 512, 384  # N = 3 heads of 128
    X = dev(workloads.llama_activations(M, K, seed=3))
    W = dev(workloads.llama_weights_bf16(N, K, seed=3).view(np.int16)).view(torch.bfloat16)
    bh, _, eb = heal.heal_split(W, residual=False)
    ah, al, ea = heal.heal_split(X)
    c = heal.heal_gemm_comp(ah, al, ea, bh, None, eb)
    q, s = heal.heal_qkv_quant_i16(c.view(M, 3, 128))
    B, L, Hq, Hkv = 2, 1000, 8, 2
    kc, ksc = workloads.int16_cache_device(B, L, Hkv, 128, seed=4)
    vc, vsc = workloads.int16_cache_device(B, L, Hkv, 128, seed=5)
    qd, qsd = (dev(a) for a in workloads.int16_cache_host(B, 1, Hq, 128, seed=6))
    out = torch.empty((B, 1, Hq, 128), dtype=torch.float32, device="cuda")
    args = heal.make_attn_args(qd, qsd, kc, ksc, vc, vsc, out, True)
    ws = torch.empty(heal.heal_attn_workspace_bytes(args), dtype=torch.uint8, device="cuda")

    def path():
        heal.heal_split(X, hi=ah, lo=al, exps=ea)
        heal.heal_gemm_comp(ah, al, ea, bh, None, eb, c=c)
        heal.heal_qkv_quant_i16(c.view(M, 3, 128), q=q, scale=s)
        heal.heal_attn_dual_fp16(qd, qsd, kc, ksc, vc, vsc, causal=True, out=out, workspace=ws)

    path()
    torch.cuda.synchronize()
    want = [t.clone() for t in (ah, al, ea, c, q, s, out)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as torch recommends before capture
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (ah, al, c, q, s, out):  # clobber the outputs eagerly between replays
            t.fill_(7 if t.dtype != torch.float32 else float("nan"))
        ea.fill_(-99)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for w, t in zip(want, (ah, al, ea, c, q, s, out)):
            assert torch.equal(w.view(torch.uint8) if w.dtype == torch.float32 else w,
                               t.view(torch.uint8) if t.dtype == torch.float32 else t), f"replay {rep}"


def test_splitk_and_fp32a_graph_replays_equal_eager(heal):
    """the split-K GEMM (caller workspace, clobbered with NaN between replays: its contents on entry do not
    matter) and the FP32-A path (row exponents + split in the GEMM) under capture"""
    banner("graph capture: split-K gemm + row exponents + FP32-A gemm, 4 replays")
    M, K, N = 128, 4096, 1024
    X = dev(workloads.llama_activations(M, K, seed=7))
    W = dev(workloads.llama_weights_bf16(N, K, seed=7).view(np.int16)).view(torch.bfloat16)
    bh, _, eb = heal.heal_split(W, residual=False)
    ah, al, ea = heal.heal_split(X)
    assert heal.heal_gemm_comp_splitk_slices(M, N, K, 2) >= 2
    ws = torch.empty(heal.heal_gemm_comp_workspace_bytes(M, N, K, 2), dtype=torch.uint8, device="cuda")
    c1 = heal.heal_gemm_comp_splitk(ah, al, ea, bh, None, eb, workspace=ws)
    e2 = heal.heal_row_exponents(X)
    c2 = heal.heal_gemm_comp_f32a(X, e2, bh, None, eb)

    def path():
        heal.heal_gemm_comp_splitk(ah, al, ea, bh, None, eb, c=c1, workspace=ws)
        heal.heal_row_exponents(X, exps=e2)
        heal.heal_gemm_comp_f32a(X, e2, bh, None, eb, c=c2)

    path()
    torch.cuda.synchronize()
    want = [t.clone() for t in (c1, e2, c2)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    torch.cuda.synchronize()
    for rep in range(4):
        c1.fill_(float("nan"))
        c2.fill_(float("nan"))
        e2.fill_(-99)
        ws.view(torch.float32).fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for w, t in zip(want, (c1, e2, c2)):
            assert torch.equal(w.view(torch.uint8), t.view(torch.uint8)), f"replay {rep}"


def test_fp32a_splitk_graph_replays_equal_eager(heal):
    """the FP32-A split-K GEMM of a 16-row down projection (row exponents, slices into the caller workspace,
    the ordered reduction) under capture; the workspace is clobbered with NaN between replays"""
    M, K, N = 16, 14336, 1024
    banner(f"graph capture: row exponents + FP32-A split-K gemm {M}x{K}->{N}, 4 replays")
    X = dev(workloads.llama_activations(M, K, seed=8))
    W = dev(workloads.llama_weights_bf16(N, K, seed=8).view(np.int16)).view(torch.bfloat16)
    bh, _, eb = heal.heal_split(W, residual=False)
    assert heal.heal_gemm_comp_f32a_splitk_slices(M, N, K, 2) >= 2
    ws = torch.empty(heal.heal_gemm_comp_f32a_workspace_bytes(M, N, K, 2), dtype=torch.uint8, device="cuda")
    e = heal.heal_row_exponents(X)
    c = heal.heal_gemm_comp_f32a_splitk(X, e, bh, None, eb, workspace=ws)

    def path():
        heal.heal_row_exponents(X, exps=e)
        heal.heal_gemm_comp_f32a_splitk(X, e, bh, None, eb, c=c, workspace=ws)

    path()
    torch.cuda.synchronize()
    want = [t.clone() for t in (e, c)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    torch.cuda.synchronize()
    for rep in range(4):
        c.fill_(float("nan"))
        e.fill_(-99)
        ws.view(torch.float32).fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for w, t in zip(want, (e, c)):
            assert torch.equal(w.view(torch.uint8), t.view(torch.uint8)), f"replay {rep}"
