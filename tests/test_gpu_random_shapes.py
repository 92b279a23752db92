"""Parity over seeded random shapes, beyond the hand-picked ones: compensated GEMMs with P = 1, 2, 3 and
ragged M, N, K (the skinny kernel and the 128 x 128 tile kernel: these shapes stay below the tile counts at
which the 256-wide tiles are chosen, which test_gpu_gemm_tiles.py checks element by element), and attention with random batch, lengths, GQA
ratios, causal or not.  Bars as elsewhere: GEMM every element within the FP32-accumulation bound of the exact
sum of its products and normwise <= 2e-6 to the FP64 definition when the residuals are kept; attention
normwise <= 2e-6 to the FP64 attention on the dequantised inputs."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, bits, dev, host, normwise

pytestmark = pytest.mark.gpu
TOL = 2e-6


def _gemm_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([rng.integers(1, 65), rng.integers(65, 700), rng.integers(700, 1300)]))
        N = int(rng.integers(1, 1500))
        K = int(rng.integers(1, 800))
        P = int(rng.integers(1, 4))
        out.append((M, N, K, P))
    return out


@pytest.mark.parametrize("M,N,K,P", _gemm_shapes(40, 2024))
def test_gemm_random_shape(heal, M, N, K, P):
    banner(f"gemm random {M}x{N}x{K} P={P}: {heal.heal_gemm_comp_variant(M, N, K, P)}")
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=M * 7 + N * 3 + K)
    ah, al, ea = heal.heal_split(dev(A))
    bh, bl, eb = heal.heal_split(dev(Bt))
    a_lo = al if P >= 2 else None
    b_lo = bl if P == 3 else None
    C = host(heal.heal_gemm_comp(ah, a_lo, ea, bh, b_lo, eb))
    parts = [bits(ah), None if a_lo is None else bits(a_lo), host(ea), bits(bh), None if b_lo is None else bits(b_lo),
             host(eb)]
    Ce, G = oracle.gemm_emul(*parts)
    viol = np.abs(C.astype(np.float64) - Ce) - (P * K + 2) * 2.0 ** -24 * G
    assert np.all(viol <= 0), f"worst excess {viol.max():.3e}"
    if P == 3:  # both residuals kept: the FP64 definition itself
        err = normwise(C, oracle.gemm_f64(A, Bt))
        print(f"[rand] gemm {M}x{N}x{K} P=3 normwise {err:.3e}")
        assert err <= TOL


def _attn_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 3, 4, 8]))
        B = int(rng.integers(1, 3))
        Lq = int(rng.choice([1, int(rng.integers(2, 300))]))
        Lkv = int(rng.integers(max(1, Lq // 2), 700)) if Lq > 1 else int(rng.integers(1, 3000))
        out.append((B, Lq, Lkv, hkv * g, hkv, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("B,Lq,Lkv,Hq,Hkv,causal", _attn_shapes(20, 77))
def test_attn_random_shape(heal, B, Lq, Lkv, Hq, Hkv, causal):
    banner(f"attention random B={B} Lq={Lq} Lkv={Lkv} Hq={Hq} Hkv={Hkv} causal={causal}")
    q, qs = workloads.int16_cache_host(B, Lq, Hq, 128, seed=Lq + 1)
    k, ks = workloads.int16_cache_host(B, Lkv, Hkv, 128, seed=Lkv + 2)
    v, vs = workloads.int16_cache_host(B, Lkv, Hkv, 128, seed=Lkv + 3)
    out = heal.heal_attn_dual_fp16(dev(q), dev(qs), dev(k), dev(ks), dev(v), dev(vs), causal=causal)
    torch.cuda.synchronize()
    ref = oracle.attn_i16_f64(q, qs, k, ks, v, vs, causal)
    got = host(out)
    # rows with no visible key (causal, Lq > Lkv) are defined as 0 on both sides
    err = normwise(got, ref) if np.linalg.norm(ref) > 0 else float(np.abs(got).max())
    print(f"[rand] attn {B},{Lq},{Lkv},{Hq},{Hkv},{causal} normwise {err:.3e}")
    assert err <= TOL
