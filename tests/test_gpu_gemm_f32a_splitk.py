"""GPU parity of heal_gemm_comp_f32a_splitk: FP32 A split in the kernel, K cut into slices for 8..16 rows with
K >= 8192 (the FP32-A form of heal_gemm_comp_splitk).

Bars ([TS 2B Mechanism]: A's primary 16-bit value and residual formed in the kernel, the products of each slice
in one FP32 accumulator):
- the same bits as heal_split + heal_gemm_comp_splitk on the parts heal_split forms (the same slices, kernel
  arithmetic and slice-order reduction);
- every element within (P K + 2) 2^-24 G of the oracle's exact sum of those 16-bit products, and normwise
  <= 2e-6 against the FP64 definition when both residuals are kept;
- the same bits on every run;
- heal_gemm_comp_f32a itself, bit for bit and without a workspace, where it does not split: K below 8192, or
  no row exponents given."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, bits, dev, host, normwise

pytestmark = pytest.mark.gpu
TOL = 2e-6


def _fp32_a(A, K):
    """A on the device with a leading dimension that is a multiple of 4 (the ABI's alignment), K itself ragged"""
    lda = (K + 3) // 4 * 4
    return dev(np.pad(A, ((0, 0), (0, lda - K))))[:, :K]


# (M, N, K, b_lo): the Llama-3-8B down projection at 16 rows, ragged K and N (a partial last slice, a partial last
# K step, columns past N in the last block), 8 and 13 rows, both product counts
CASES = [(16, 4096, 14336, False), (16, 1000, 9001, True), (8, 300, 8200, False), (13, 520, 16390, True),
         (11, 777, 12345, False)]


@pytest.mark.parametrize("M,N,K,b_lo", CASES)
def test_f32a_splitk_equals_split_then_splitk(heal, M, N, K, b_lo):
    P = 3 if b_lo else 2
    S = heal.heal_gemm_comp_f32a_splitk_slices(M, N, K, P)
    banner(f"gemm FP32-A split-K {M}x{N}x{K} P={P} S={S}")
    assert S >= 2
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=M + N + K)
    a = _fp32_a(A, K)
    bh, bl, eb = heal.heal_split(dev(Bt))
    bl = bl if b_lo else None
    ea = heal.heal_row_exponents(a)
    c = heal.heal_gemm_comp_f32a_splitk(a, ea, bh, bl, eb)
    c2 = heal.heal_gemm_comp_f32a_splitk(a, ea, bh, bl, eb)
    ah, al, ea2 = heal.heal_split(a)
    c_ref = heal.heal_gemm_comp_splitk(ah, al, ea2, bh, bl, eb)
    torch.cuda.synchronize()
    assert torch.equal(ea, ea2)
    assert torch.equal(c.view(torch.int32), c2.view(torch.int32)), "not run-to-run deterministic"
    assert torch.equal(c.view(torch.int32), c_ref.view(torch.int32)), "differs from heal_split + splitk"
    C = host(c)
    Ce, G = oracle.gemm_emul(bits(ah), bits(al), host(ea2), bits(bh), None if bl is None else bits(bl), host(eb))
    viol = np.abs(C.astype(np.float64) - Ce) - (P * K + 2) * 2.0 ** -24 * G
    assert float(viol.max()) <= 0, f"bound violated at {np.unravel_index(viol.argmax(), viol.shape)}"
    err = normwise(C, oracle.gemm_f64(A, Bt))
    print(f"[f32a splitk] {M}x{N}x{K} P={P} S={S} normwise {err:.3e}")
    if P == 3:
        assert err <= TOL


@pytest.mark.parametrize("M,N,K,with_exps", [(16, 1000, 4096, True), (4, 1000, 9000, True),
                                             (16, 1000, 9001, False)])
def test_f32a_splitk_whole_is_f32a(heal, M, N, K, with_exps):
    """no split (K < 8192, under 8 rows, or no row exponents): heal_gemm_comp_f32a, bit for bit, no workspace"""
    banner(f"gemm FP32-A split-K kept whole {M}x{N}x{K} exponents given {with_exps}")
    if with_exps:
        assert heal.heal_gemm_comp_f32a_splitk_slices(M, N, K, 2) == 1
        assert heal.heal_gemm_comp_f32a_workspace_bytes(M, N, K, 2) == 0
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=M + K)
    a = _fp32_a(A, K)
    bh, _, eb = heal.heal_split(dev(Bt), residual=False)
    ea = heal.heal_row_exponents(a) if with_exps else None
    c = heal.heal_gemm_comp_f32a_splitk(a, ea, bh, None, eb)
    c_ref = heal.heal_gemm_comp_f32a(a, ea, bh, None, eb)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int32), c_ref.view(torch.int32))


def test_f32a_splitk_llama_down_bf16_weights(heal):
    """the decode-batch down projection 16 x 14336 -> 4096 with bf16 N(0, 0.02) weights (exact in one FP16 part
    after the column prescale: P = 2), sampled against FP64"""
    M, K, N = 16, 14336, 4096
    banner(f"gemm FP32-A split-K llama down {M}x{K}->{N}")
    X = workloads.llama_activations(M, K, seed=9)
    W = workloads.llama_weights_bf16(N, K, seed=9)
    bh, _, eb = heal.heal_split(dev(W.view(np.int16)).view(torch.bfloat16), residual=False)
    x = dev(X)
    c = heal.heal_gemm_comp_f32a_splitk(x, heal.heal_row_exponents(x), bh, None, eb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    ii, jj = rng.integers(0, M, 2048), rng.integers(0, N, 2048)
    ref = oracle.gemm_f64_points(X.astype(np.float64), oracle.part_values(W, oracle.BF16), ii, jj)
    err = normwise(host(c)[ii, jj], ref)
    print(f"[f32a splitk] llama down sampled normwise {err:.3e}")
    assert err <= TOL
