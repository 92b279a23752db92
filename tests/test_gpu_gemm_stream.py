"""Element-wise GPU parity of the streamed-B kernel (gemm_stream_kernel) that serves at most 16 rows when N gives
every CU a column block of 16, the CUs' blocks times K's stages of 128 come to at least 64 per CU, and A's split
parts fit in LDS: each persistent workgroup walks several
column blocks, and each block's 16 rows of B stream through a ring of direct-to-LDS stages of 128 of K.

Covered: both A sources (16-bit parts, and FP32 rows split in the kernel with given or derived row exponents),
P = 1, 2, 3 (B's low part shortens the ring), FP16 and bf16 parts, ragged K (a partial last stage with
K % 8 != 0, whose part padding holds NaN patterns), N not a multiple of 16 (rows past N), and 1 to 16 rows.

Bar ([TS 2B Mechanism]: the products of the 16-bit parts are summed in one FP32 accumulator): every element within
|C - C_e| <= (P K + 2) 2^-24 G of the oracle's exact sum C_e of the same 16-bit products; normwise <= 2e-6
against the FP64 definition where the kept products represent the operands exactly; and heal_gemm_comp_f32a equal
to heal_split + heal_gemm_comp bit for bit (the same kernel on the same parts)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, bits, dev, host, normwise

pytestmark = pytest.mark.gpu
TOL = 2e-6


def _wide_n(heal, M, K, P, extra):
    """the smallest N (plus `extra`) for which the variant is the stream kernel"""
    for N in range(16, 1 << 17, 16):
        if heal.heal_gemm_comp_variant(M, N + extra, K, P).startswith("gemm_stream_kernel"):
            return N + extra
    raise AssertionError("no N selects the stream kernel")


def _bound(C, ah, al, ea, bh, bl, eb, K, P, part):
    parts = [bits(ah), None if al is None else bits(al), None if ea is None else host(ea), bits(bh),
             None if bl is None else bits(bl), None if eb is None else host(eb)]
    Ce, G = oracle.gemm_emul(*parts, part=oracle.F16 if part == "f16" else oracle.BF16)
    viol = np.abs(C.astype(np.float64) - Ce) - (P * K + 2) * 2.0 ** -24 * G
    assert float(viol.max()) <= 0, f"bound violated at {np.unravel_index(viol.argmax(), viol.shape)}"


# (M, K, a_lo, b_lo, part): 4 ring stages per wavefront, 2 with B's low part
CASES = [
    (1, 1000, True, False, "f16"), (3, 4001, True, False, "f16"), (16, 100 * 8 + 5, True, False, "f16"),
    (1, 9000, True, False, "f16"), (1, 9000, True, True, "f16"), (2, 1003, True, True, "f16"),
    (1, 4001, False, False, "f16"), (5, 1000, False, True, "f16"), (1, 9000, True, True, "bf16"),
]


@pytest.mark.parametrize("M,K,a_lo,b_lo,part", CASES)
def test_stream_parts_elementwise(heal, M, K, a_lo, b_lo, part):
    P = 1 + a_lo + b_lo
    N = _wide_n(heal, M, K, 3 if b_lo else P, extra=5)  # rows past N in the last block
    banner(f"gemm stream {M}x{N}x{K} P={P} {part}")
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=M + K + P)
    prescale = part == "f16"
    ah, al, ea = heal.heal_split(dev(A), part=part, prescale=prescale)
    bh, bl, eb = heal.heal_split(dev(Bt), part=part, prescale=prescale)
    # NaN patterns (0xFFFF) in the padding columns past K of every part row must not reach the sums
    for t in (ah, al, bh, bl):
        ld = t.stride(0)
        if ld > K:
            torch.as_strided(t, (t.shape[0], ld), (ld, 1))[:, K:] = -1
    al, bl = (al if a_lo else None), (bl if b_lo else None)
    ea, eb = (ea, eb) if prescale else (None, None)
    C = host(heal.heal_gemm_comp(ah, al, ea, bh, bl, eb, part=part))
    _bound(C, ah, al, ea, bh, bl, eb, K, P, part)
    if P == 3 and part == "f16":
        err = normwise(C, oracle.gemm_f64(A, Bt))
        print(f"[stream] {M}x{N}x{K} P=3 normwise {err:.3e}")
        assert err <= TOL


@pytest.mark.parametrize("M,K,b_lo,derived", [(1, 4096, False, True), (1, 4096, False, False),
                                               (16, 800, True, True), (1, 14336, False, True),
                                               (4, 2001, True, False)])
def test_stream_f32a_equals_split_then_gemm(heal, M, K, b_lo, derived):
    """heal_gemm_comp_f32a (A split in the kernel) against heal_split + heal_gemm_comp: the same bits"""
    P = 3 if b_lo else 2
    N = _wide_n(heal, M, K, P, extra=3)
    banner(f"gemm stream FP32 A {M}x{N}x{K} P={P} derived exponents {derived}")
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=7 + M + K)
    # FP32 rows with a leading dimension that is a multiple of 4 (the ABI's alignment), K itself ragged
    lda = (K + 3) // 4 * 4
    a = dev(np.pad(A, ((0, 0), (0, lda - K))))[:, :K]
    bh, bl, eb = heal.heal_split(dev(Bt))
    bl = bl if b_lo else None
    ah, al, ea = heal.heal_split(a)
    c_ref = heal.heal_gemm_comp(ah, al, ea, bh, bl, eb)
    c = heal.heal_gemm_comp_f32a(a, None if derived else heal.heal_row_exponents(a), bh, bl, eb)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int32), c_ref.view(torch.int32))
    _bound(host(c), ah, al, ea, bh, bl, eb, K, P, "f16")


def test_stream_llama_gate_up_sampled(heal):
    """the decode step's fused gate/up projection, one row: 1 x 4096 -> 28672 with bf16 weights, sampled against
    FP64, and twice the same bits"""
    M, K, N = 1, 4096, 28672
    assert heal.heal_gemm_comp_variant(M, N, K, 2).startswith("gemm_stream_kernel")
    banner(f"gemm stream llama gate/up {M}x{N}x{K}")
    X = workloads.llama_activations(M, K, seed=3)
    W = workloads.llama_weights_bf16(N, K, seed=3)
    bh, _, eb = heal.heal_split(dev(W.view(np.int16)).view(torch.bfloat16), residual=False)
    x = dev(X)
    c1 = heal.heal_gemm_comp_f32a(x, None, bh, None, eb)
    c2 = heal.heal_gemm_comp_f32a(x, None, bh, None, eb)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))
    jj = np.random.default_rng(0).integers(0, N, 2048)
    ref = oracle.gemm_f64_points(X.astype(np.float64), oracle.part_values(W, oracle.BF16), np.zeros(2048, int), jj)
    err = normwise(host(c1)[0, jj], ref)
    print(f"[stream] gate/up sampled normwise {err:.3e}")
    assert err <= TOL
