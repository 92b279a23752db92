"""The largest sizes: tensors past 2^31 elements, so every offset must be 64-bit.  Each case reads or writes
elements beyond element 2^31 and checks them: sampled outputs against the oracle (GEMM, split, quantiser), and
for decode a cache built so that the exact answer is known in closed form at any size."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, bits, dev, host, normwise

pytestmark = pytest.mark.gpu
TOL = 2e-6
BIG = 1 << 31


def test_gemm_output_past_2_31_elements(heal):
    M, N, K = 65539, 32773, 40  # C: 2.148e9 elements; rows >= 65522 start past element 2^31
    banner(f"large gemm {M}x{N}x{K} P=3: {heal.heal_gemm_comp_variant(M, N, K, 3)}")
    A, Bt = workloads.gemm_uniform(M, N, K, seed=11)
    ah, al, ea = heal.heal_split(dev(A))
    bh, bl, eb = heal.heal_split(dev(Bt))
    C = heal.heal_gemm_comp(ah, al, ea, bh, bl, eb)
    torch.cuda.synchronize()
    assert C.shape[0] * C.stride(0) > BIG
    rng = np.random.default_rng(11)
    ii = np.concatenate([[0, M // 2, 65521, 65522, 65530, M - 1] * 8, rng.integers(0, M, 464)])
    jj = np.concatenate([np.repeat([0, 1, N // 2, N - 2, N - 1, 7, 31000, 32000], 6), rng.integers(0, N, 464)])
    got = host(C[torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()])
    ref = oracle.gemm_f64_points(A, Bt, ii, jj)
    err = normwise(got, ref)
    print(f"[large] gemm sampled normwise {err:.3e}")
    assert err <= TOL
    assert torch.isfinite(C).all()
    del C, ah, al, bh, bl
    torch.cuda.empty_cache()


def test_split_rows_past_2_31_elements(heal):
    rows, cols = (1 << 21) + 7, 1032  # 2.164e9 elements
    banner(f"large split {rows}x{cols}")
    g = torch.Generator(device="cuda").manual_seed(12)
    x = torch.randn((rows, cols), device="cuda", generator=g) * 3.0
    hi, lo, e = heal.heal_split(x)
    torch.cuda.synchronize()
    sel = np.array([0, 1, rows // 2, (BIG // cols) - 1, BIG // cols, BIG // cols + 1, rows - 2, rows - 1])
    xs = host(x[torch.from_numpy(sel).cuda()])
    ohi, olo, oe = oracle.split_f32(xs)
    s = torch.from_numpy(sel).cuda()
    assert np.array_equal(bits(hi[s]), ohi)
    assert np.array_equal(bits(lo[s]), olo)
    assert np.array_equal(host(e[s]), oe)
    del x, hi, lo, e
    torch.cuda.empty_cache()


def test_quant_rows_past_2_31_elements(heal):
    tokens, heads, D = (1 << 20) + 5, 16, 128  # 2.1475e9 elements
    banner(f"large quantiser {tokens}x{heads}x{D}")
    g = torch.Generator(device="cuda").manual_seed(13)
    x = torch.randn((tokens, heads, D), device="cuda", generator=g)
    q, s = heal.heal_qkv_quant_i16(x)
    torch.cuda.synchronize()
    sel = np.array([0, tokens // 2, BIG // (heads * D) - 1, BIG // (heads * D), tokens - 1])
    t = torch.from_numpy(sel).cuda()
    oq, os_ = oracle.quant_i16(host(x[t]))
    assert np.array_equal(host(q[t]), oq)
    assert np.array_equal(host(s[t]).view(np.uint32), os_.view(np.uint32))
    del x, q, s
    torch.cuda.empty_cache()


def test_decode_cache_past_2_31_elements(heal):
    """One sequence of L keys, 8 KV heads (K and V 2.1475e9 elements each).  Keys 0 .. 2^21 - 1 are zero and
    the last 64 (all past element 2^31) hold 100 in every component, as does the query, so their logit
    exceeds every other by more than 2^17 and every other weight is exactly 0, while the 64 of them tie at
    weight 1.  The output is then exactly the mean of those 64 value rows (integers, scales 1)."""
    B, Hq, Hkv, D = 1, 8, 8, 128
    L = (1 << 21) + 64
    banner(f"large decode L={L} Hkv={Hkv}")
    k = torch.zeros((B, L, Hkv, D), dtype=torch.int16, device="cuda")
    v = torch.zeros((B, L, Hkv, D), dtype=torch.int16, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(14)
    v[:, : L - 64] = torch.randint(-300, 300, (B, L - 64, Hkv, D), device="cuda", generator=g,
                                   dtype=torch.int16)
    k[:, L - 64:] = 100
    tail = torch.randint(-20000, 20000, (B, 64, Hkv, D), device="cuda", generator=g, dtype=torch.int16)
    v[:, L - 64:] = tail
    assert k[0, L - 64:].data_ptr() - k.data_ptr() >= 2 * BIG  # the tail's first element is past 2^31
    ks = torch.ones((B, L, Hkv), dtype=torch.float32, device="cuda")
    vs = torch.ones((B, L, Hkv), dtype=torch.float32, device="cuda")
    q = torch.full((B, 1, Hq, D), 100, dtype=torch.int16, device="cuda")
    qs = torch.ones((B, 1, Hq), dtype=torch.float32, device="cuda")
    out = heal.heal_attn_dual_fp16(q, qs, k, ks, v, vs, causal=True)
    torch.cuda.synchronize()
    want = host(tail.to(torch.float64)).mean(axis=1)  # [B, Hkv, D]; G = 1
    got = host(out)[:, 0]
    assert np.abs(got - want).max() <= 1e-6 * np.abs(want).max(), f"max diff {np.abs(got - want).max():.3e}"
    del k, v, ks, vs, tail, out
    torch.cuda.empty_cache()
