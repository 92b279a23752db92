"""GPU parity of the fused GEMM + INT16 quantisation (heal_gemm_comp_quant_i16).

Bar: for M > 64 the codes and scales equal heal_gemm_comp followed by heal_qkv_quant_i16 bit for bit, and
equal the oracle's quantiser applied to the GPU's C (so the epilogue follows the quantisation rule itself,
not only the GPU quantiser).  For M <= 64 (a different GEMM kernel than heal_gemm_comp's skinny one) every
code is within one step of the two-step path and the dequantised output is within the quantisation bound of
the FP64 product."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, bits, dev, host

pytestmark = pytest.mark.gpu


def _parts(heal, M, N, K, P, seed=0):
    A, Bt = workloads.gemm_uniform(M, N, K, seed=seed)
    ah, al, ea = heal.heal_split(dev(A))
    bh, bl, eb = heal.heal_split(dev(Bt), residual=(P == 3))
    return A, Bt, (ah, al, ea, bh, bl if P == 3 else None, eb)


@pytest.mark.parametrize("M,N,K,P", [
    (2048, 8192, 256, 3),   # 256 x 256 tiles: a head is one wavefront's 128 columns
    (2048, 4096, 512, 2),   # 128 x 256 tiles: a head is one wavefront's 128 columns
    (2048, 4096, 512, 3),   # 256 x 128 tiles: a head spans two wavefronts (row maxima meet in LDS)
    (300, 384, 200, 3),     # 128 x 128 tiles, ragged M
    (129, 256, 1000, 2),
])
def test_fused_quant_equals_gemm_then_quant(heal, M, N, K, P):
    banner(f"gemm+quant fused {M}x{N}x{K} P={P}")
    _, _, parts = _parts(heal, M, N, K, P)
    c = heal.heal_gemm_comp(*parts)
    q2, s2 = heal.heal_qkv_quant_i16(c.contiguous().view(M, N // 128, 128))
    q1, s1 = heal.heal_gemm_comp_quant_i16(*parts)
    torch.cuda.synchronize()
    assert np.array_equal(host(q1), host(q2).reshape(M, N))
    assert np.array_equal(host(s1).view(np.uint32), host(s2).view(np.uint32))
    # the oracle's quantiser on the GPU's C gives the same codes and scales
    qo, so = oracle.quant_i16(host(c).reshape(M, N // 128, 128))
    assert np.array_equal(host(q1), qo.reshape(M, N)) and np.array_equal(host(s1), so)


def test_fused_quant_into_a_larger_cache(heal):
    banner("gemm+quant fused into a strided cache view")
    M, N, K = 256, 512, 384
    _, _, parts = _parts(heal, M, N, K, 3, seed=2)
    cache = torch.full((M, N + 256), 7, dtype=torch.int16, device="cuda")
    scales = torch.full((M, 8), -1.0, dtype=torch.float32, device="cuda")
    q1, s1 = heal.heal_gemm_comp_quant_i16(*parts, q=cache[:, 128:128 + N], scale=scales[:, 2:2 + N // 128])
    q2, s2 = heal.heal_gemm_comp_quant_i16(*parts)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
    # nothing outside the views was written
    assert bool((cache[:, :128] == 7).all()) and bool((cache[:, 128 + N:] == 7).all())
    assert bool((scales[:, :2] == -1).all()) and bool((scales[:, 2 + N // 128:] == -1).all())


def test_fused_quant_small_m(heal):
    banner("gemm+quant fused, M = 16 (tile kernel) against the skinny two-step path and FP64")
    M, N, K = 16, 1024, 4096
    X = workloads.llama_activations(M, K, seed=3)
    W = workloads.llama_weights_bf16(N, K, seed=3)
    bh, _, eb = heal.heal_split(dev(W.view(np.int16)).view(torch.bfloat16), residual=False)
    ah, al, ea = heal.heal_split(dev(X))
    parts = (ah, al, ea, bh, None, eb)
    q1, s1 = heal.heal_gemm_comp_quant_i16(*parts)
    c = heal.heal_gemm_comp(*parts)
    q2, s2 = heal.heal_qkv_quant_i16(c.contiguous().view(M, N // 128, 128))
    torch.cuda.synchronize()
    d = np.abs(host(q1).astype(np.int32) - host(q2).reshape(M, N).astype(np.int32))
    assert d.max() <= 1
    # both C's are within the FP32 accumulation bound (P K + 2) 2^-24 G of the exact sum of the same
    # products, so their row maxima per head differ by at most twice that, and the scales by that / 32767
    # plus one rounding each
    Ce, G = oracle.gemm_emul(bits(ah), bits(al), host(ea), bits(bh), None, host(eb))
    dc = (2 * (2 * K + 2) * 2.0 ** -24 * G).reshape(M, N // 128, 128).max(-1)
    s1h, s2h = host(s1).astype(np.float64), host(s2).reshape(M, N // 128).astype(np.float64)
    assert np.all(np.abs(s1h - s2h) <= dc / 32767 + 2.0 ** -23 * np.maximum(s1h, s2h))
    # dequantised codes against the FP64 product: within half a step (plus the GEMM's own error)
    ref = oracle.gemm_f64(X.astype(np.float64), oracle.part_values(W, oracle.BF16))
    s = np.repeat(host(s1).astype(np.float64), 128, axis=1)
    err = np.abs(host(q1).astype(np.float64) * s - ref)
    assert np.all(err <= s * (0.5 + 2.0 ** -9) + 1e-5 * np.abs(ref).max())
