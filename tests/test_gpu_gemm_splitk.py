"""GPU parity of the split-K compensated GEMM (heal_gemm_comp_splitk) against the oracle.

Same bars as heal_gemm_comp: every element within the FP32-accumulation bound (P K + 2) 2^-24 G of the exact
sum of its 16-bit products (splitting K regroups the FP32 additions, which only lowers that worst case), and
normwise <= 2e-6 against the FP64 definition when both residuals are kept.  Also: the same bits on every run,
the plan's slice counts, and heal_gemm_comp itself, bit for bit, where the plan does not split."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, bits, dev, host, normwise

pytestmark = pytest.mark.gpu
TOL = 2e-6


def _parts(heal, A, Bt, a_residual=True, b_residual=True):
    ah, al, ea = heal.heal_split(dev(A), residual=a_residual)
    bh, bl, eb = heal.heal_split(dev(Bt), residual=b_residual)
    return ah, al, ea, bh, bl, eb


def _bound_check(C, parts, K):
    ah, al, ea, bh, bl, eb = [None if p is None else (bits(p) if p.dtype == torch.int16 else host(p))
                              for p in parts]
    P = 1 + (al is not None) + (bl is not None)
    Ce, G = oracle.gemm_emul(ah, al, ea, bh, bl, eb)
    viol = np.abs(C.astype(np.float64) - Ce) - (P * K + 2) * 2.0 ** -24 * G
    assert np.all(viol <= 0), f"per-element bound violated, worst excess {viol.max():.3e}"


# tile and skinny splits, ragged K (a partial last slice and a partial last K step), each product count
@pytest.mark.parametrize("M,N,K,P", [
    (100, 300, 5001, 3), (129, 257, 4100, 2), (300, 200, 2100, 1),      # 128 x 128 tiles, K split
    (40, 1000, 3001, 3), (64, 500, 4096, 2), (20, 700, 2003, 3),        # 17..64-row skinny, K split
    (16, 1000, 9001, 3), (8, 300, 8200, 2), (13, 520, 16390, 1)])       # 8..16 rows, K >= 8192
def test_splitk_bound_and_fp64(heal, M, N, K, P):
    S = heal.heal_gemm_comp_splitk_slices(M, N, K, P)
    banner(f"gemm split-K {M}x{N}x{K} P={P} S={S}")
    assert S >= 2
    A, Bt = workloads.gemm_uniform(M, N, K, seed=M + K)
    parts = _parts(heal, A, Bt, a_residual=P >= 2, b_residual=P == 3)
    C = heal.heal_gemm_comp_splitk(*parts)
    C2 = heal.heal_gemm_comp_splitk(*parts)
    torch.cuda.synchronize()
    C, C2 = host(C), host(C2)
    assert np.array_equal(C.view(np.uint32), C2.view(np.uint32)), "split-K is not run-to-run deterministic"
    _bound_check(C, parts, K)
    if P == 3:
        err = normwise(C, oracle.gemm_f64(A, Bt))
        print(f"[splitk] {M}x{N}x{K} S={S} normwise {err:.3e}")
        assert err <= TOL


def test_splitk_bf16_parts(heal):
    """the bf16 contrast parts go through the same split kernels"""
    M, N, K = 100, 300, 3000
    banner(f"gemm split-K bf16 parts {M}x{N}x{K}")
    A, Bt = workloads.gemm_uniform(M, N, K, seed=5)
    ah, al, _ = heal.heal_split(dev(A), part="bf16", prescale=False)
    bh, bl, _ = heal.heal_split(dev(Bt), part="bf16", prescale=False)
    assert heal.heal_gemm_comp_splitk_slices(M, N, K, 3) >= 2
    c_split = host(heal.heal_gemm_comp_splitk(ah, al, None, bh, bl, None, part="bf16"))
    c_plain = host(heal.heal_gemm_comp(ah, al, None, bh, bl, None, part="bf16"))
    Ce, G = oracle.gemm_emul(bits(ah), bits(al), None, bits(bh), bits(bl), None, part=oracle.BF16)
    for C in (c_split, c_plain):
        viol = np.abs(C.astype(np.float64) - Ce) - (3 * K + 2) * 2.0 ** -24 * G
        assert np.all(viol <= 0)


@pytest.mark.parametrize("M,N,K", [(16, 4096, 4096), (1024, 4096, 1000), (2048, 4096, 512)])
def test_no_split_is_heal_gemm_comp(heal, M, N, K):
    """where the plan keeps K whole the call is heal_gemm_comp, bit for bit, without a workspace"""
    banner(f"gemm split-K plan S=1 {M}x{N}x{K}")
    assert heal.heal_gemm_comp_splitk_slices(M, N, K, 2) == 1
    assert heal.heal_gemm_comp_workspace_bytes(M, N, K, 2) == 0
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=3)
    ah, al, ea, bh, _, eb = _parts(heal, A, Bt, b_residual=False)
    c1 = heal.heal_gemm_comp_splitk(ah, al, ea, bh, None, eb)
    c2 = heal.heal_gemm_comp(ah, al, ea, bh, None, eb)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))


@pytest.mark.parametrize("M", [16, 32, 64, 128, 512])
@pytest.mark.parametrize("K,N", workloads.LLAMA3_8B_KN)
def test_llama_medium_m_sampled(heal, M, K, N):
    """medium-M Llama-3-8B projections (decode batches, short prefills), sampled against FP64"""
    S = heal.heal_gemm_comp_splitk_slices(M, N, K, 2)
    banner(f"gemm split-K llama M={M} K={K} N={N} S={S}")
    X = workloads.llama_activations(M, K, seed=2)
    W = workloads.llama_weights_bf16(N, K, seed=2)
    bh, _, eb = heal.heal_split(dev(W.view(np.int16)).view(torch.bfloat16), residual=False)
    ah, al, ea = heal.heal_split(dev(X))
    C = heal.heal_gemm_comp_splitk(ah, al, ea, bh, None, eb)
    Cp = heal.heal_gemm_comp(ah, al, ea, bh, None, eb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M + K + N)
    ii, jj = rng.integers(0, M, 512), rng.integers(0, N, 512)
    ref = oracle.gemm_f64_points(X.astype(np.float64), oracle.part_values(W, oracle.BF16), ii, jj)
    err = normwise(host(C)[ii, jj], ref)
    err_p = normwise(host(Cp)[ii, jj], ref)
    print(f"[splitk] llama M={M} K={K} N={N} S={S} sampled normwise {err:.3e} (unsplit {err_p:.3e})")
    assert err <= TOL
    assert torch.isfinite(C).all()
