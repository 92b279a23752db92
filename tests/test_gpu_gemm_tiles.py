"""Element-wise GPU parity of every block-tile kernel the compensated GEMM dispatches to, at shapes where that
tile is the one chosen: 256 x 256 (P = 1, 2, 3, FP16 and bf16 parts), 128 x 256 (P = 2), 256 x 128 (P = 1, 3)
and the fused INT16-quantising variants of 256 x 256, 128 x 256 and 256 x 128.

Each case asserts the kernel by name (heal_gemm_comp_variant), uses ragged M and N (partial edge tiles) and K
of several hundred (K % 32 != 0, so the steady-state loop over full K tiles runs many times before the partial
last tile, and K % 8 != 0 where the padding columns of a part row must be ignored).

Bar ([TS 2B Mechanism]: the products of the 16-bit parts are summed in one FP32 accumulator):
  * every element within the FP32-accumulation bound |C - C_e| <= (P K + 2) 2^-24 G of the oracle's exact sum
    C_e of the same 16-bit products (G the sum of their magnitudes);
  * where the kept products represent the operands exactly (P = 3, or P = 2 with 16-bit-exact B), normwise
    relative error <= 2e-6 against the FP64 definition C* = A B;
  * fused quantisation: codes and scales equal to the oracle's quantiser applied to heal_gemm_comp's C (which
    passes the bound above), bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, bits, dev, host, normwise

pytestmark = pytest.mark.gpu
TOL = 2e-6


def _operands(M, N, K, b_exact16, seed):
    """A fp32 with rows scaled by 10^U(-3, 3); B^T fp32 the same way, or bf16-valued weights (exact in FP16 after
    the row prescale) when b_exact16."""
    A, Bt = workloads.gemm_rowscaled(M, N, K, seed=seed)
    if b_exact16:
        w = workloads.llama_weights_bf16(N, K, seed=seed)
        Bt = (w.astype(np.uint32) << 16).view(np.float32)
    return A, Bt


def _check_bound(C, ah, al, ea, bh, bl, eb, K, P, part):
    parts = [bits(ah), None if al is None else bits(al), host(ea) if ea is not None else None, bits(bh),
             None if bl is None else bits(bl), host(eb) if eb is not None else None]
    Ce, G = oracle.gemm_emul(*parts, part=oracle.F16 if part == "f16" else oracle.BF16)
    viol = np.abs(C.astype(np.float64) - Ce) - (P * K + 2) * 2.0 ** -24 * G
    worst = float(viol.max())
    assert worst <= 0, f"per-element bound violated at {np.unravel_index(viol.argmax(), viol.shape)}, excess {worst:.3e}"


# (M, N, K, a_lo, b_lo, part, expected kernel)
CASES = [
    (4000, 4100, 610, True, True, "f16", "gemm_comp_kernel 256x256 P3"),
    (4000, 4100, 600, True, False, "f16", "gemm_comp_kernel 256x256 P2"),
    (4000, 4100, 330, False, False, "f16", "gemm_comp_kernel 256x256 P1"),
    (4000, 4100, 330, True, True, "bf16", "gemm_comp_kernel 256x256 P3"),
    (2050, 4100, 610, True, False, "f16", "gemm_comp_kernel 128x256 P2"),
    (2050, 4100, 610, True, True, "f16", "gemm_comp_kernel 256x128 P3"),
    (2050, 4100, 330, False, False, "f16", "gemm_comp_kernel 256x128 P1"),
    (2050, 4100, 330, False, True, "f16", "gemm_comp_kernel 256x128 P2"),
]


@pytest.mark.parametrize("M,N,K,a_lo,b_lo,part,kernel", CASES)
def test_tile_kernel_elementwise(heal, M, N, K, a_lo, b_lo, part, kernel):
    P = 1 + a_lo + b_lo
    # heal_gemm_comp_variant's products = 2 names the A-low-part case; B's low part alone runs the P = 2
    # instantiation of the choice made without the 128 x 256 option
    if P == 2 and b_lo:
        name = heal.heal_gemm_comp_variant(M, N, K, 3).replace("P3", "P2")
    else:
        name = heal.heal_gemm_comp_variant(M, N, K, P)
    assert name == kernel, name
    banner(f"gemm tile {M}x{N}x{K} P={P} {part}: {kernel}")
    exact16 = (P == 2 and a_lo) and part == "f16"
    A, Bt = _operands(M, N, K, exact16, seed=M + N + K + P)
    prescale = part == "f16"
    ah, al, ea = heal.heal_split(dev(A), part=part, prescale=prescale)
    bh, bl, eb = heal.heal_split(dev(Bt), part=part, prescale=prescale)
    al, bl = (al if a_lo else None), (bl if b_lo else None)
    C = host(heal.heal_gemm_comp(ah, al, ea if prescale else None, bh, bl, eb if prescale else None, part=part))
    _check_bound(C, ah, al, ea if prescale else None, bh, bl, eb if prescale else None, K, P, part)
    if part == "f16" and (P == 3 or exact16):
        err = normwise(C, oracle.gemm_f64(A, Bt))
        print(f"[tile] {kernel} {M}x{N}x{K} normwise {err:.3e}")
        assert err <= TOL


# fused INT16 quantisation of C per (row, 128-column head): (M, N, K, P, expected kernel)
QUANT_CASES = [
    (4000, 4224, 610, 3, "gemm_comp_kernel 256x256 P3"),
    (2050, 4096, 610, 2, "gemm_comp_kernel 128x256 P2"),
    (2050, 4096, 610, 3, "gemm_comp_kernel 256x128 P3"),
]


@pytest.mark.parametrize("M,N,K,P,kernel", QUANT_CASES)
def test_tile_kernel_fused_quant(heal, M, N, K, P, kernel):
    assert heal.heal_gemm_comp_variant(M, N, K, P) == kernel
    banner(f"gemm+quant tile {M}x{N}x{K} P={P}: {kernel}")
    A, Bt = _operands(M, N, K, P == 2, seed=3 * M + N + K)
    ah, al, ea = heal.heal_split(dev(A))
    bh, bl, eb = heal.heal_split(dev(Bt), residual=(P == 3))
    parts = (ah, al, ea, bh, bl if P == 3 else None, eb)
    c = heal.heal_gemm_comp(*parts)
    q1, s1 = heal.heal_gemm_comp_quant_i16(*parts)
    torch.cuda.synchronize()
    C = host(c)
    _check_bound(C, ah, al, ea, bh, parts[4], eb, K, P, "f16")
    qo, so = oracle.quant_i16(C.reshape(M, N // 128, 128))
    assert np.array_equal(host(q1), qo.reshape(M, N))
    assert np.array_equal(host(s1).view(np.uint32), so.view(np.uint32))
