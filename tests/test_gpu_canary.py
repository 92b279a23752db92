"""Canary bands: every output is written into a view of a larger buffer whose other bytes hold a sentinel
pattern (0x7FA5A5A5, a NaN), and must leave them untouched while the view equals, bit for bit, the output
written into a plain allocation.  Covers the GEMM kernels (skinny, skinny with A split in LDS, the persistent
streamed-B kernel, 128 x 128, 128 x 256, 256 x 256 with three products, split K, the 16-row split-K streamed-B
kernel and its workspace), the split's part padding, the quantiser writing into a
cache view, and prefill and decode attention writing a strided output."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import banner, dev

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FA5A5A5


def _guarded(rows, cols, dtype, pad_rows=2, pad_cols=12):
    """a buffer of sentinel bits with pad_rows rows above and below and pad_cols columns left of and (at least)
    right of a [rows, cols] interior view; the row length is rounded up to 16 bytes, as leading dimensions
    must be"""
    per16 = 16 // torch.empty((), dtype=dtype).element_size()
    width = (cols + per16 - 1) // per16 * per16 + 2 * pad_cols
    n = torch.empty((rows + 2 * pad_rows, width), dtype=dtype, device="cuda")
    n.view(torch.int32 if n.element_size() == 4 else torch.int16).fill_(
        SENTINEL if n.element_size() == 4 else np.int16(np.uint16(0xA5A5).astype(np.int16)))
    return n, n[pad_rows:pad_rows + rows, pad_cols:pad_cols + cols]


def _outside_untouched(buf, view):
    mask = torch.ones(buf.shape, dtype=torch.bool, device="cuda")
    r0 = (view.data_ptr() - buf.data_ptr()) // buf.element_size() // buf.stride(0)
    c0 = (view.data_ptr() - buf.data_ptr()) // buf.element_size() % buf.stride(0)
    mask[r0:r0 + view.shape[0], c0:c0 + view.shape[1]] = False
    raw = buf.view(torch.int32 if buf.element_size() == 4 else torch.int16)
    want = SENTINEL if buf.element_size() == 4 else int(np.uint16(0xA5A5).astype(np.int16))
    return bool((raw[mask] == want).all())


@pytest.mark.parametrize("P,f32a", [(2, False), (3, False), (2, True)])
def test_stream_splitk_writes_only_its_view_and_workspace(heal, P, f32a):
    """the 16-row split-K launch (gemm_stream_sk_kernel writing each slice's partials into the caller workspace,
    then the ordered reduction) into a strided view: the view's guard bands and a sentinel band past the end of
    the workspace stay untouched, and the view equals the same call into a plain allocation"""
    M, N, K = 16, 1003, 9000
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=6)
    ah, al, ea = heal.heal_split(dev(A))
    bh, bl, eb = heal.heal_split(dev(Bt), residual=(P == 3))
    bl = bl if P == 3 else None
    a = dev(np.pad(A, ((0, 0), (0, (K + 3) // 4 * 4 - K))))[:, :K]
    if f32a:
        S, need = heal.heal_gemm_comp_f32a_splitk_slices(M, N, K, P), heal.heal_gemm_comp_f32a_workspace_bytes(M, N, K, P)
    else:
        S, need = heal.heal_gemm_comp_splitk_slices(M, N, K, P), heal.heal_gemm_comp_workspace_bytes(M, N, K, P)
    banner(f"canary stream split-K {M}x{N}x{K} P={P} f32a={f32a} S={S}")
    assert S > 1 and need == S * M * ((N + 3) // 4 * 4) * 4
    wsbuf = torch.empty(need // 4 + 4096, dtype=torch.int32, device="cuda")
    wsbuf.fill_(SENTINEL)
    ws = wsbuf[:need // 4].view(torch.uint8)
    run = ((lambda c: heal.heal_gemm_comp_f32a_splitk(a, heal.heal_row_exponents(a), bh, bl, eb, c=c, workspace=ws))
           if f32a else (lambda c: heal.heal_gemm_comp_splitk(ah, al, ea, bh, bl, eb, c=c, workspace=ws)))
    ref = run(None)  # the binding's own output (rows padded to 16 bytes)
    buf, view = _guarded(M, N, torch.float32, pad_cols=4)
    run(view)
    torch.cuda.synchronize()
    assert bool((wsbuf[need // 4:] == SENTINEL).all()), "written past the workspace"
    assert _outside_untouched(buf, view)
    assert torch.equal(view.contiguous().view(torch.int32), ref.contiguous().view(torch.int32))


@pytest.mark.parametrize("M,N,K,P,f32a", [(1, 4100, 1032, 2, True), (16, 3000, 777, 3, False), (300, 520, 300, 3, False),
                                        (2050, 4100, 96, 2, False), (4000, 4100, 64, 3, False), (100, 600, 4096, 2, False),
                                        (3, 12300, 1000, 2, True), (5, 12300, 1000, 3, False)])
def test_gemm_writes_only_its_view(heal, M, N, K, P, f32a):
    banner(f"canary gemm {M}x{N}x{K} P={P} f32a={f32a}: {heal.heal_gemm_comp_variant(M, N, K, P)}")
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=5)
    ah, al, ea = heal.heal_split(dev(A))
    bh, bl, eb = heal.heal_split(dev(Bt), residual=(P == 3))
    bl = bl if P == 3 else None
    buf, view = _guarded(M, N, torch.float32, pad_cols=4)  # interior starts 16 bytes in, ldc = N + 8
    if f32a:
        ref = heal.heal_gemm_comp_f32a(dev(A), None, bh, bl, eb)
        heal.heal_gemm_comp_f32a(dev(A), None, bh, bl, eb, c=view)
    else:
        ref = heal.heal_gemm_comp(ah, al, ea, bh, bl, eb)
        heal.heal_gemm_comp(ah, al, ea, bh, bl, eb, c=view)
    torch.cuda.synchronize()
    assert _outside_untouched(buf, view)
    assert torch.equal(view.contiguous().view(torch.int32), ref.contiguous().view(torch.int32))
    if M == 100:  # the split-K launch (partials in a workspace, then the ordered reduction) into the same view
        ws = torch.empty(max(heal.heal_gemm_comp_workspace_bytes(M, N, K, P), 256), dtype=torch.uint8, device="cuda")
        buf2, view2 = _guarded(M, N, torch.float32, pad_cols=4)
        heal.heal_gemm_comp_splitk(ah, al, ea, bh, bl, eb, c=view2, workspace=ws)
        torch.cuda.synchronize()
        assert heal.heal_gemm_comp_splitk_slices(M, N, K, P) > 1
        assert _outside_untouched(buf2, view2)


def test_split_and_quant_write_only_their_views(heal):
    banner("canary split parts and quantiser cache view")
    x = dev(workloads.gemm_rowscaled(33, 1, 4100, seed=6)[0])  # A [33, 4100]
    for cols in (100, 4100):
        hb, hv = _guarded(33, cols, torch.int16, pad_cols=8)
        lb, lv = _guarded(33, cols, torch.int16, pad_cols=8)
        h0, l0, e0 = heal.heal_split(x[:, :cols].contiguous())
        heal.heal_split(x[:, :cols].contiguous(), hi=hv, lo=lv)
        torch.cuda.synchronize()
        assert _outside_untouched(hb, hv) and _outside_untouched(lb, lv)
        assert torch.equal(hv, h0) and torch.equal(lv, l0)
    Q = dev(workloads.qkv_fp32(1, 70, 6, 128, seed=3)[0][0])  # [70, 6, 128]
    qb, qv = _guarded(70, 6 * 128, torch.int16, pad_cols=8)
    sb, sv = _guarded(70, 6, torch.float32, pad_cols=4)
    q0, s0 = heal.heal_qkv_quant_i16(Q)
    heal.heal_qkv_quant_i16(Q, q=qv.view(70, 6, 128), scale=sv)
    torch.cuda.synchronize()
    assert _outside_untouched(qb, qv) and _outside_untouched(sb, sv)
    assert torch.equal(qv.reshape(70, 6, 128), q0) and torch.equal(sv, s0)


@pytest.mark.parametrize("Lq", [1, 150])
def test_attention_writes_only_its_view(heal, Lq):
    banner(f"canary attention output, q_len {Lq}")
    B, L, Hq, Hkv = 2, 300, 4, 2
    q, qs = workloads.int16_cache_host(B, Lq, Hq, 128, seed=8)
    k, ks = workloads.int16_cache_host(B, L, Hkv, 128, seed=9)
    v, vs = workloads.int16_cache_host(B, L, Hkv, 128, seed=10)
    args = [dev(t) for t in (q, qs, k, ks, v, vs)]
    ref = heal.heal_attn_dual_fp16(*args, causal=True)
    # each head's 128 outputs sit in a 160-wide slot, with sentinel rows of tokens before and after
    buf = torch.empty((B, Lq + 2, Hq, 160), dtype=torch.float32, device="cuda")
    buf.view(torch.int32).fill_(SENTINEL)
    out = buf[:, 1:1 + Lq, :, 16:144]
    heal.heal_attn_dual_fp16(*args, causal=True, out=out)
    torch.cuda.synchronize()
    inside = torch.zeros(buf.shape, dtype=torch.bool, device="cuda")
    inside[:, 1:1 + Lq, :, 16:144] = True
    assert bool((buf.view(torch.int32)[~inside] == SENTINEL).all())
    assert torch.equal(out.contiguous().view(torch.int32), ref.view(torch.int32))
