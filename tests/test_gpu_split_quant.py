"""GPU parity of the HBM-bound passes against the oracle: bit-exact split (FP32/bf16 -> FP16/bf16 parts
with the power-of-two row prescale), Dual-FP16 INT16 unpack and INT16 quantisation."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, bits, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 7), (5, 8), (17, 1000), (256, 256), (64, 14336), (2048, 4096),
                                       # rows held in registers (2049 .. 16384 columns), ragged, and just past
                                       (9, 2049), (7, 8195), (5, 16383), (4, 16384), (3, 16385)])
def test_split_f32_f16_bit_exact(heal, rows, cols):
    banner(f"split f32->f16 {rows}x{cols}")
    rng = np.random.default_rng(rows * 1000 + cols)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-6, 6, size=(rows, 1))).astype(np.float32)
    if rows > 2:
        x[1] = 0.0
        x[2, :: 3] *= np.float32(1e-30)  # residuals that fall into fp16 subnormals / fp32 subnormals
    hi, lo, e = heal.heal_split(dev(x))
    torch.cuda.synchronize()
    ohi, olo, oe = oracle.split_f32(x)
    assert np.array_equal(host(e), oe)
    assert np.array_equal(bits(hi), ohi)
    assert np.array_equal(bits(lo), olo)


def test_split_modes(heal):
    banner("split modes: no prescale, no residual, bf16 parts, bf16 input")
    rng = np.random.default_rng(1)
    for cols in (203, 4100):  # the two-pass kernel and the row-in-registers one
        x = (rng.standard_normal((37, cols)) * 3).astype(np.float32)
        x[0, 0] = 7e4  # overflows fp16 without the prescale
        for part, p in (("f16", oracle.F16), ("bf16", oracle.BF16)):
            for pre in (True, False):
                for res in (True, False):
                    hi, lo, e = heal.heal_split(dev(x), part=part, prescale=pre, residual=res)
                    torch.cuda.synchronize()
                    ohi, olo, oe = oracle.split_f32(x, part=p, prescale=pre, residual=res)
                    assert np.array_equal(bits(hi), ohi), (cols, part, pre, res)
                    if res:
                        assert np.array_equal(bits(lo), olo), (cols, part, pre, res)
                    if pre:
                        assert np.array_equal(host(e), oe)
    W = workloads.llama_weights_bf16(96, 4104, seed=5)  # ragged cols
    wt = dev(W.view(np.int16)).view(torch.bfloat16)
    hi, lo, e = heal.heal_split(wt, residual=False)
    torch.cuda.synchronize()
    ohi, _, oe = oracle.split_bf16(W)
    assert np.array_equal(bits(hi), ohi) and np.array_equal(host(e), oe)


def test_split_i16_exhaustive(heal):
    banner("split i16 all 65536 values")
    q = np.arange(-32768, 32768, dtype=np.int32).astype(np.int16).reshape(256, 256)
    hi, lo, _ = heal.heal_split(dev(q))
    torch.cuda.synchronize()
    ohi, olo = oracle.split_i16(q)
    assert np.array_equal(bits(hi), ohi) and np.array_equal(bits(lo), olo)
    q2 = q[:5, :13].copy()  # ragged
    hi, lo, _ = heal.heal_split(dev(q2))
    torch.cuda.synchronize()
    ohi, olo = oracle.split_i16(q2)
    assert np.array_equal(bits(hi), ohi) and np.array_equal(bits(lo), olo)


@pytest.mark.parametrize("T,H,D", [(256, 1, 128), (300, 8, 128), (4096, 32, 128), (33, 3, 64), (7, 2, 256),
                                   (5, 1, 1024), (9, 4, 4),
                                   (4096, 96, 128)])  # Q, K and V heads of a token side by side, one launch
def test_quant_bit_exact(heal, T, H, D):
    banner(f"quant {T}x{H}x{D}")
    x, _, _ = workloads.qkv_fp32(1, T, H, D, seed=T + H + D)
    x = x[0]
    if T > 4:
        x[3, 0] = 0.0
        x[4, 0, :] = np.float32(1e-39) * np.sign(x[4, 0, :])  # subnormal scale
    q, s = heal.heal_qkv_quant_i16(dev(x))
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_i16(x)
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(host(q), oq)


def test_quant_ties_and_cache_append(heal):
    banner("quant ties + strided cache append")
    k = -10
    row = np.zeros((1, 1, 8), np.float32)
    row[0, 0, 0] = 32767.0 * 2.0 ** k
    row[0, 0, 1:] = np.array([2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5]) * 2.0 ** k
    q, s = heal.heal_qkv_quant_i16(dev(row))
    assert list(host(q)[0, 0]) == [32767, 2, 4, -2, -4, 0, 2, 0]
    # quantise 3 new tokens per sequence straight into a [B, S_max, H, D] cache at position 5
    B, Smax, H, D = 2, 16, 4, 128
    cache = torch.zeros((B, Smax, H, D), dtype=torch.int16, device="cuda")
    sc = torch.zeros((B, Smax, H), dtype=torch.float32, device="cuda")
    x, _, _ = workloads.qkv_fp32(B, 3, H, D, seed=4)
    for b in range(B):
        heal.heal_qkv_quant_i16(dev(x[b]), q=cache[b, 5:8], scale=sc[b, 5:8])
    torch.cuda.synchronize()
    for b in range(B):
        oq, os_ = oracle.quant_i16(x[b])
        assert np.array_equal(host(cache[b, 5:8]), oq) and np.array_equal(host(sc[b, 5:8]), os_)
    assert int(cache[:, :5].abs().sum()) == 0 and int(cache[:, 8:].abs().sum()) == 0
