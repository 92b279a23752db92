"""Pins of the oracle's GEMM levels.

Definition level (FP64 C = A B): reduces to numpy's float64 matmul (library routine) and to exact
rational arithmetic on tiny inputs.  Emulation level (exact sum of the method's 16-bit products,
[TS 2B Mechanism]; [TS] = gist.science explainer "Demystifying Numerical Instability in LLM Inference ...
with HEAL", Technical Summary): pinned by closed-form error bounds of the split (so a dropped product, a
wrong sign or a transposed operand fails), exact integer special cases and K = 1."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads


def test_definition_matches_numpy_float64():
    rng = np.random.default_rng(0)
    for M, N, K in ((1, 1, 1), (7, 5, 3), (33, 17, 65), (64, 48, 200)):
        A = rng.standard_normal((M, K))
        Bt = rng.standard_normal((N, K))
        C = oracle.gemm_f64(A, Bt)
        R = A @ Bt.T
        assert np.allclose(C, R, rtol=1e-13, atol=1e-13 * (np.abs(A) @ np.abs(Bt).T).max())
        ii = rng.integers(0, M, 9)
        jj = rng.integers(0, N, 9)
        assert np.allclose(oracle.gemm_f64_points(A, Bt, ii, jj), R[ii, jj], rtol=1e-13, atol=1e-12)


def test_definition_bruteforce_exact_rationals():
    rng = np.random.default_rng(1)
    A = rng.standard_normal((4, 6)).astype(np.float32).astype(np.float64)
    Bt = rng.standard_normal((5, 6)).astype(np.float32).astype(np.float64)
    C = oracle.gemm_f64(A, Bt)
    for i in range(4):
        for j in range(5):
            exact = sum(Fraction(A[i, k]) * Fraction(Bt[j, k]) for k in range(6))
            assert abs(Fraction(C[i, j]) - exact) <= Fraction(6 * 2.0 ** -52) * sum(
                abs(Fraction(A[i, k]) * Fraction(Bt[j, k])) for k in range(6))


def _split_both(A, Bt):
    ah, al, ea = oracle.split_f32(A)
    bh, bl, eb = oracle.split_f32(Bt)
    return ah, al, ea, bh, bl, eb


@pytest.mark.parametrize("gen", ["uniform", "rowscaled"])
def test_emulation_within_split_bound(gen):
    M, N, K = 48, 40, 96
    if gen == "uniform":
        A, Bt = workloads.gemm_uniform(M, N, K, seed=0)
    else:
        A, Bt = workloads.gemm_rowscaled(M, N, K, seed=4)
    ah, al, ea, bh, bl, eb = _split_both(A, Bt)
    Ce, G = oracle.gemm_emul(ah, al, ea, bh, bl, eb)
    Cs = oracle.gemm_f64(A.astype(np.float64), Bt.astype(np.float64))
    absAB = np.abs(A.astype(np.float64)) @ np.abs(Bt.astype(np.float64)).T
    # each operand is reproduced by hi + lo within 2^-22 of its row's scaled value (11 + 11 bits), the
    # dropped lo*lo term is below 2^-22 of |a||b|: 4 * 2^-22 |A||B| bounds the emulation's departure
    err = np.abs(Ce - Cs)
    assert np.all(err <= 4 * 2.0 ** -22 * absAB + 1e-300)
    # ... and the bound is not vacuous: the products matter at the 2^-11 level
    Ce1, _ = oracle.gemm_emul(ah, None, ea, bh, None, eb)
    assert np.max(np.abs(Ce1 - Cs) / absAB) > 2.0 ** -14
    # G is the magnitude sum of the same products: >= |C_e| and close to |A||B|
    assert np.all(G >= np.abs(Ce) * (1 - 1e-15))
    assert np.allclose(G, absAB, rtol=2.0 ** -9)


def test_emulation_two_products_for_exact_weights():
    X = workloads.llama_activations(8, 256, seed=1)
    W = workloads.llama_weights_bf16(24, 256, seed=1)
    xh, xl, ex = oracle.split_f32(X)
    wh, _, ew = oracle.split_bf16(W)
    Ce, _ = oracle.gemm_emul(xh, xl, ex, wh, None, ew)
    Wd = oracle.part_values(W, oracle.BF16)
    Cs = oracle.gemm_f64(X.astype(np.float64), Wd)
    absAB = np.abs(X.astype(np.float64)) @ np.abs(Wd).T
    assert np.all(np.abs(Ce - Cs) <= 2 * 2.0 ** -22 * absAB)


def test_emulation_integer_inputs_exact():
    rng = np.random.default_rng(2)
    A = rng.integers(-8, 9, (20, 1024)).astype(np.float32)
    Bt = rng.integers(-8, 9, (12, 1024)).astype(np.float32)
    A[3] = 0.0
    ah, al, ea, bh, bl, eb = _split_both(A, Bt)
    assert np.all(oracle.part_values(al, oracle.F16) == 0)
    Ce, _ = oracle.gemm_emul(ah, al, ea, bh, bl, eb)
    exact = A.astype(np.int64) @ Bt.astype(np.int64).T
    assert np.array_equal(Ce, exact.astype(np.float64))


def test_emulation_k1_and_transpose_sensitivity():
    rng = np.random.default_rng(7)
    a = rng.standard_normal((9, 1)).astype(np.float32)
    b = rng.standard_normal((11, 1)).astype(np.float32)
    ah, al, ea, bh, bl, eb = _split_both(a, b)
    Ce, _ = oracle.gemm_emul(ah, al, ea, bh, bl, eb)
    ref = a.astype(np.float64) @ b.astype(np.float64).T
    assert np.all(np.abs(Ce - ref) <= 2.0 ** -21 * np.abs(ref))
    # a non-square case: swapping operand roles gives the transpose, not the same matrix
    A, Bt = workloads.gemm_uniform(5, 7, 9, seed=3)
    C1, _ = oracle.gemm_emul(*_split_both(A, Bt))
    C2, _ = oracle.gemm_emul(*_split_both(Bt, A))
    assert np.allclose(C1, C2.T, rtol=0, atol=1e-12) and C1.shape == (5, 7)
