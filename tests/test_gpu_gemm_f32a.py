"""GPU parity of the GEMM that splits its FP32 A operand in the prologue (heal_row_exponents +
heal_gemm_comp_f32a, [TS 2B Mechanism]).

Bar: the row exponents equal heal_split's bit for bit; C equals heal_split + heal_gemm_comp bit for bit
(the same parts, MFMAs and accumulation order) on every kernel kind (skinny with 1, 2 and 4 column
blocks, 128 x 128, 128 x 256, 256 x 128 and 256 x 256 tiles, 2 and 3 products) with ragged M, N and K,
including K not a multiple of 4; and against the oracle: normwise <= 2e-6 to the FP64 definition and
every element within the FP32-accumulation bound of the exact sum of the same products."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, bits, dev, host, normwise

pytestmark = pytest.mark.gpu
TOL = 2e-6


def _a_dev(A):
    """FP32 A on the device with a leading dimension rounded up to 4 floats, as a [M, K] view"""
    M, K = A.shape
    t = torch.zeros((M, (K + 3) // 4 * 4), dtype=torch.float32, device="cuda")
    t[:, :K] = dev(A)
    return t[:, :K]


def _both(heal, A, Bt, b_residual):
    a = _a_dev(A)
    bh, bl, eb = heal.heal_split(dev(Bt), residual=b_residual)
    ah, al, ea = heal.heal_split(a)
    c_ref = heal.heal_gemm_comp(ah, al, ea, bh, bl, eb)
    e2 = heal.heal_row_exponents(a)
    c = heal.heal_gemm_comp_f32a(a, e2, bh, bl, eb)
    torch.cuda.synchronize()
    assert torch.equal(e2, ea)
    return host(c), host(c_ref), (ah, al, ea, bh, bl, eb)


@pytest.mark.parametrize("M,N,K,P", [
    (1, 300, 77, 2), (16, 7300, 130, 2), (30, 7300, 301, 3), (64, 1000, 1001, 2), (5, 14350, 64, 3),   # skinny
    (30, 14390, 70, 2), (30, 14390, 70, 3), (50, 7300, 130, 2), (64, 14390, 77, 2),                     # NC 2, 4
    (64, 14390, 77, 3),                           # three products at 64 rows: NC 1 against split + GEMM's NC 4
    (16, 777, 1016, 2), (16, 777, 1024, 3),       # A's split planes just fit the 64 KB of LDS / just do not
    (100, 300, 1003, 2), (129, 257, 999, 3),                                                            # 128 x 128
    (2048, 4096, 258, 2),                                                                               # 128 x 256
    (2048, 4096, 130, 3),                                                                               # 256 x 128
    (2048, 14336, 97, 2), (2048, 14336, 66, 3)])                                                        # 256 x 256
def test_fused_equals_split_then_gemm(heal, M, N, K, P):
    banner(f"gemm f32a {M}x{N}x{K} P={P}: {heal.heal_gemm_comp_variant(M, N, K, P)}")
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=7)
    c, c_ref, _ = _both(heal, A, Bt, b_residual=(P == 3))
    assert np.array_equal(c.view(np.uint32), c_ref.view(np.uint32))


@pytest.mark.parametrize("M,N,K", [(300, 200, 1001), (16, 1000, 777)])
def test_fused_vs_oracle(heal, M, N, K):
    banner(f"gemm f32a vs oracle {M}x{N}x{K} P=3")
    A, Bt = workloads.gemm_uniform(M, N, K, seed=3)
    c, _, parts = _both(heal, A, Bt, b_residual=True)
    ah, al, ea, bh, bl, eb = [bits(p) if p.dtype == torch.int16 else host(p) for p in parts]
    Ce, G = oracle.gemm_emul(ah, al, ea, bh, bl, eb)
    assert np.all(np.abs(c.astype(np.float64) - Ce) <= (3 * K + 2) * 2.0 ** -24 * G)
    err = normwise(c, oracle.gemm_f64(A, Bt))
    print(f"[f32a] {M}x{N}x{K} normwise {err:.3e}")
    assert err <= TOL


def test_row_exponents_special_rows(heal):
    banner("row exponents: zero row, subnormal maximum, empty rows")
    x = np.random.default_rng(1).standard_normal((6, 37)).astype(np.float32)
    x[1] = 0
    x[2] = np.float32(1e-40)  # subnormal maximum
    x[3, 5] = np.float32(3e38)
    xd = dev(x)
    e = heal.heal_row_exponents(xd)
    _, _, es = heal.heal_split(xd)
    torch.cuda.synchronize()
    assert torch.equal(e, es)
    assert host(e)[1] == 0
    e0 = heal.heal_row_exponents(xd[:, :0])
    torch.cuda.synchronize()
    assert np.all(host(e0) == 0)


@pytest.mark.parametrize("M", [1, 16, 2048])
@pytest.mark.parametrize("K,N", workloads.LLAMA3_8B_KN)
def test_llama_linear_fused(heal, M, K, N):
    """every Llama-3-8B projection at the bench's sizes (its decode-sized shapes run this entry point)"""
    banner(f"gemm f32a llama M={M} K={K} N={N}")
    X = workloads.llama_activations(M, K, seed=1)
    W = workloads.llama_weights_bf16(N, K, seed=1)
    bh, _, eb = heal.heal_split(dev(W.view(np.int16)).view(torch.bfloat16), residual=False)
    a = _a_dev(X)
    ah, al, ea = heal.heal_split(a)
    c_ref = heal.heal_gemm_comp(ah, al, ea, bh, None, eb)
    c = heal.heal_gemm_comp_f32a(a, heal.heal_row_exponents(a), bh, None, eb)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int32), c_ref.view(torch.int32))
    rng = np.random.default_rng(M + K)
    ii, jj = rng.integers(0, M, 256), rng.integers(0, N, 256)
    ref = oracle.gemm_f64_points(X.astype(np.float64), oracle.part_values(W, oracle.BF16), ii, jj)
    err = normwise(host(c)[ii, jj], ref)
    print(f"[f32a] llama M={M} K={K} N={N} sampled normwise {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("M,N,K,P", [(1, 300, 77, 2), (1, 14336, 4096, 2), (1, 4096, 14336, 2), (3, 700, 1001, 3),
                                     (16, 4096, 4096, 2), (16, 14350, 130, 3), (5, 300, 3, 2), (4, 7300, 64, 2),
                                     (16, 777, 1016, 3), (16, 777, 1024, 2), (2, 3000, 8184, 2)])
def test_derived_row_exponents(heal, M, N, K, P):
    """a_exp = None (at most 16 rows): the kernel derives the row exponents itself, so C is bit for bit what the
    exponents of heal_row_exponents give.  Rows with no nonzero value, a subnormal maximum and a value near
    1e30 are included, and the padding past K holds 1e30, which would change an exponent if it were read."""
    banner(f"gemm f32a derived exponents {M}x{N}x{K} P={P}")
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=11)
    if M >= 3:
        A[0] = 0.0
        A[1] = np.float32(1e-40) * np.sign(A[1] + 0.5)
        A[2, K // 2] = np.float32(1e30)
    t = torch.full((M, (K + 3) // 4 * 4 + 4), 1e30, dtype=torch.float32, device="cuda")
    t[:, :K] = dev(A)
    a = t[:, :K]
    bh, bl, eb = heal.heal_split(dev(Bt), residual=(P == 3))
    c_given = heal.heal_gemm_comp_f32a(a, heal.heal_row_exponents(a), bh, bl, eb)
    c_derived = heal.heal_gemm_comp_f32a(a, None, bh, bl, eb)
    torch.cuda.synchronize()
    assert torch.equal(c_derived.view(torch.int32), c_given.view(torch.int32))
    assert bool(torch.isfinite(c_derived).all())


def test_derived_row_exponents_refused_above_16_rows(heal):
    a = torch.zeros((17, 64), dtype=torch.float32, device="cuda")
    bh, _, eb = heal.heal_split(torch.ones((32, 64), dtype=torch.float32, device="cuda"), residual=False)
    with pytest.raises(RuntimeError):
        heal.heal_gemm_comp_f32a(a, None, bh, None, eb)
