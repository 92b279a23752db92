"""GPU parity of the compensated GEMM against the oracle.

Bar: normwise relative error <= 2e-6 against the FP64 definition C* = A B; every element within the
FP32-accumulation bound |C - C_e| <= (P K + 2) 2^-24 G of the emulation (C_e the exact sum of the same P K
16-bit products, G the sum of their magnitudes: n rounded additions of partial sums bounded by G); exact
special cases bit for bit; run-to-run bit determinism."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, bits, dev, host, normwise

pytestmark = pytest.mark.gpu
TOL = 2e-6


def _split_dev(heal, x, residual=True):
    return heal.heal_split(dev(x), residual=residual)


def _gemm_full(heal, A, Bt, b_residual=True):
    ah, al, ea = _split_dev(heal, A)
    bh, bl, eb = _split_dev(heal, Bt, residual=b_residual)
    C = heal.heal_gemm_comp(ah, al, ea, bh, bl, eb)
    torch.cuda.synchronize()
    return host(C), (ah, al, ea, bh, bl, eb)


def _bound_check(C, parts, K):
    ah, al, ea, bh, bl, eb = [None if p is None else (bits(p) if p.dtype == torch.int16 else host(p))
                              for p in parts]
    P = 1 + (al is not None) + (bl is not None)
    Ce, G = oracle.gemm_emul(ah, al, ea, bh, bl, eb)
    viol = np.abs(C.astype(np.float64) - Ce) - (P * K + 2) * 2.0 ** -24 * G
    assert np.all(viol <= 0), f"per-element bound violated, worst excess {viol.max():.3e}"
    return Ce


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (1, 1, 1), (7, 5, 3), (300, 200, 100), (129, 257, 1000),
                                   (64, 640, 4104), (513, 96, 33), (20, 70, 999), (48, 33, 64), (65, 300, 130),
                                   # skinny workgroups of 2 and 4 column blocks with ragged N and K
                                   (3, 7201, 130), (16, 14350, 77), (30, 7300, 300),
                                   # 32- and 64-row skinny workgroups with 2 and 4 column blocks
                                   (30, 14390, 70), (50, 7300, 130), (64, 14390, 77)])
def test_uniform_p3(heal, M, N, K):
    banner(f"gemm uniform P=3 {M}x{N}x{K}")
    A, Bt = workloads.gemm_uniform(M, N, K, seed=0)
    C, parts = _gemm_full(heal, A, Bt)
    Cs = oracle.gemm_f64(A, Bt)
    _bound_check(C, parts, K)
    err = normwise(C, Cs)
    print(f"[gemm] {M}x{N}x{K} P=3 normwise {err:.3e}")
    assert err <= TOL


def test_rowscaled_p3_and_bf16_contrast(heal):
    banner("gemm rowscaled P=3 1024x768x512 + bf16 contrast")
    M, N, K = 1024, 768, 512
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=4)
    C, parts = _gemm_full(heal, A, Bt)
    Cs = oracle.gemm_f64(A, Bt)
    _bound_check(C, parts, K)
    err = normwise(C, Cs)
    absAB = np.abs(A.astype(np.float64)) @ np.abs(Bt.astype(np.float64)).T
    comp = float(np.max(np.abs(C - Cs) / absAB))
    print(f"[gemm] rowscaled normwise {err:.3e} componentwise {comp:.3e}")
    assert err <= TOL and comp <= 1e-6
    # contrast: bf16 parts (3 products, no prescale) and plain bf16 (1 product)
    ah, al, _ = heal.heal_split(dev(A), part="bf16", prescale=False)
    bh, bl, _ = heal.heal_split(dev(Bt), part="bf16", prescale=False)
    c3 = host(heal.heal_gemm_comp(ah, al, None, bh, bl, None, part="bf16"))
    c1 = host(heal.heal_gemm_comp(ah, None, None, bh, None, None, part="bf16"))
    e3, e1 = normwise(c3, Cs), normwise(c1, Cs)
    print(f"[gemm] bf16x3 contrast {e3:.3e}  plain bf16 {e1:.3e}")
    assert 1e-7 < e3 < 5e-5 and 1e-4 < e1 < 1e-2


def test_integer_inputs_exact(heal):
    banner("gemm integer inputs exact")
    rng = np.random.default_rng(2)
    A = rng.integers(-8, 9, (200, 1024)).astype(np.float32)
    Bt = rng.integers(-8, 9, (136, 1024)).astype(np.float32)
    A[7] = 0
    C, _ = _gemm_full(heal, A, Bt)
    exact = (A.astype(np.int64) @ Bt.astype(np.int64).T).astype(np.float32)
    assert np.array_equal(C, exact)


def test_fp16_exact_inputs_equal_one_product(heal):
    banner("gemm lo = 0 -> equals P=1")
    rng = np.random.default_rng(3)
    A = rng.integers(-1024, 1024, (96, 320)).astype(np.float32) * np.float32(2.0 ** -7)
    Bt = rng.integers(-1024, 1024, (80, 320)).astype(np.float32) * np.float32(2.0 ** -3)
    ah, al, ea = _split_dev(heal, A)
    bh, bl, eb = _split_dev(heal, Bt)
    assert int(al.abs().sum()) == 0 and int(bl.abs().sum()) == 0
    c3 = host(heal.heal_gemm_comp(ah, al, ea, bh, bl, eb))
    c1 = host(heal.heal_gemm_comp(ah, None, ea, bh, None, eb))
    assert np.array_equal(c3, c1)


def test_k_zero_and_determinism(heal):
    banner("gemm K=0, determinism")
    z = torch.zeros((5, 8), dtype=torch.int16, device="cuda")[:, :0]
    C = heal.heal_gemm_comp(z, None, None, torch.zeros((3, 8), dtype=torch.int16, device="cuda")[:, :0], None,
                            None)
    torch.cuda.synchronize()
    assert np.all(host(C) == 0)
    A, Bt = workloads.gemm_rowscaled(640, 520, 700, seed=9)
    C1, _ = _gemm_full(heal, A, Bt)
    C2, _ = _gemm_full(heal, A, Bt)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))


@pytest.mark.parametrize("M", [1, 16, 2048])
@pytest.mark.parametrize("K,N", workloads.LLAMA3_8B_KN)
def test_llama_linear_p2_sampled(heal, M, K, N):
    banner(f"gemm llama linear P=2 M={M} K={K} N={N}")
    X = workloads.llama_activations(M, K, seed=1)
    W = workloads.llama_weights_bf16(N, K, seed=1)
    wt = dev(W.view(np.int16)).view(torch.bfloat16)
    bh, _, eb = heal.heal_split(wt, residual=False)
    ah, al, ea = heal.heal_split(dev(X))
    C = heal.heal_gemm_comp(ah, al, ea, bh, None, eb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M + K + N)
    ii = rng.integers(0, M, 512)
    jj = rng.integers(0, N, 512)
    Wd = oracle.part_values(W, oracle.BF16)
    ref = oracle.gemm_f64_points(X.astype(np.float64), Wd, ii, jj)
    got = host(C)[ii, jj]
    err = normwise(got, ref)
    print(f"[gemm] llama M={M} K={K} N={N} sampled normwise {err:.3e}")
    assert err <= TOL
    # full-matrix property at any size: no NaN/Inf
    assert torch.isfinite(C).all()


def test_config5_8192_sampled(heal):
    banner("gemm 8192^3 rowscaled P=3 sampled")
    M = N = K = 8192
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=4)
    ah, al, ea = heal.heal_split(dev(A))
    bh, bl, eb = heal.heal_split(dev(Bt))
    C = heal.heal_gemm_comp(ah, al, ea, bh, bl, eb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    ii = rng.integers(0, M, 1024)
    jj = rng.integers(0, N, 1024)
    ref = oracle.gemm_f64_points(A.astype(np.float64), Bt.astype(np.float64), ii, jj)
    got = host(C)[ii, jj]
    err = normwise(got, ref)
    print(f"[gemm] 8192^3 sampled normwise {err:.3e}")
    assert err <= TOL
    # 24 whole rows (every column, the launch the bench times) element by element against the oracle's exact
    # sum of the same 16-bit products, within the FP32-accumulation bound (3 K + 2) 2^-24 G
    rows = np.sort(rng.choice(M, 24, replace=False))
    Ce, G = oracle.gemm_emul(bits(ah)[rows], bits(al)[rows], host(ea)[rows], bits(bh), bits(bl), host(eb))
    viol = np.abs(host(C)[rows].astype(np.float64) - Ce) - (3 * K + 2) * 2.0 ** -24 * G
    assert float(viol.max()) <= 0, f"per-element bound violated, excess {viol.max():.3e}"
