"""GPU parity of the calibrated outlier channels (heal_channel_exponents, heal_split_scaled).

Bar: exponents and split bits equal the oracle's bit for bit (integer decisions and exact power-of-two
scaling, taken in fp32 on both sides); end to end, on massive-activation inputs the calibrated GEMM is within
2e-6 normwise of the FP64 product on the outputs made of ordinary values, where the uncalibrated one is not."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import bits, dev, host, banner, normwise

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,T", [(2048, 4096, -12), (301, 1000, -12), (7, 65, 0), (1, 8, -140 + 20)])
def test_channel_exponents_exact(heal, M, K, T):
    banner(f"channel exponents {M}x{K} T={T}")
    x, _ = workloads.massive_channels(M, K, seed=M + K)
    got = host(heal.heal_channel_exponents(dev(x), T))
    assert np.array_equal(got, oracle.channel_exponents(x, T))


def test_channel_exponents_strided_rows(heal):
    x, _ = workloads.massive_channels(300, 640, seed=5)
    big = torch.zeros((300, 700), dtype=torch.float32, device="cuda")
    big[:, :640] = dev(x)
    got = host(heal.heal_channel_exponents(big[:, :640], -10))
    assert np.array_equal(got, oracle.channel_exponents(x, -10))


@pytest.mark.parametrize("M,K", [(256, 4096), (64, 14336), (17, 5004), (33, 1003), (5, 7)])
def test_split_scaled_exact(heal, M, K):
    banner(f"split scaled {M}x{K}")
    x, _ = workloads.massive_channels(M, K, seed=7)
    c = oracle.channel_exponents(x, -12)
    cd = dev(c)
    hi, lo, e = heal.heal_split_scaled(dev(x), cd, +1)
    oh, ol, oe = oracle.split_f32(oracle.scale_columns(x, c, +1))
    assert np.array_equal(bits(hi), oh) and np.array_equal(bits(lo), ol) and np.array_equal(host(e), oe)
    # bf16 weights, scaled the other way
    w = workloads.llama_weights_bf16(64, K, seed=8)
    wt = dev(w.view(np.int16)).view(torch.bfloat16)
    bh, _, eb = heal.heal_split_scaled(wt, cd, -1, residual=False)
    wh, _, we = oracle.split_f32(oracle.scale_columns(oracle.part_values(w, oracle.BF16), c, -1), residual=False)
    assert np.array_equal(bits(bh), wh) and np.array_equal(host(eb), we)
    # rows that do not start 16-byte aligned take the element-by-element path
    xs = torch.zeros((M, K + 1), dtype=torch.float32, device="cuda")
    xs[:, 1:] = dev(x)
    h2, l2, e2 = heal.heal_split_scaled(xs[:, 1:], cd, +1)
    assert np.array_equal(bits(h2), oh) and np.array_equal(bits(l2), ol) and np.array_equal(host(e2), oe)


def test_massive_channels_end_to_end(heal):
    banner("massive channels: calibrated vs plain compensated GEMM, 256x4096x512")
    M, K, N = 256, 4096, 512
    x, idx = workloads.massive_channels(M, K, seed=11)
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[: N // 2][:, idx] = 0.0  # the first half of the outputs never sees the massive channels
    ref = oracle.gemm_f64(x.astype(np.float64), w.astype(np.float64))
    xd, wd = dev(x), dev(w)
    half = slice(0, N // 2)
    c = heal.heal_channel_exponents(xd, -12)
    ah, al, ea = heal.heal_split_scaled(xd, c, +1)
    bh, bl, eb = heal.heal_split_scaled(wd, c, -1)
    cal = host(heal.heal_gemm_comp(ah, al, ea, bh, bl, eb))
    ah0, al0, ea0 = heal.heal_split(xd)
    bh0, bl0, eb0 = heal.heal_split(wd)
    plain = host(heal.heal_gemm_comp(ah0, al0, ea0, bh0, bl0, eb0))
    e_cal, e_plain = normwise(cal[:, half], ref[:, half]), normwise(plain[:, half], ref[:, half])
    print(f"[channels] ordinary outputs: calibrated {e_cal:.3e}, plain {e_plain:.3e}; "
          f"all outputs calibrated {normwise(cal, ref):.3e}")
    assert e_cal <= 2e-6 and e_plain > 1e-4
    assert normwise(cal, ref) <= 2e-6
