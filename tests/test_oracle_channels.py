"""Pins of the oracle's calibrated outlier channels ([TS 2B Overflow Handling]: targeted rescaling of rare
outlier channels, read as exact power-of-two column scales folded into the weights; [TS] = gist.science
explainer "Demystifying Numerical Instability in LLM Inference ... with HEAL", Technical Summary).

Pins: hand-worked exponents; every scaled column's maximum lands below 2^(T+1) and unscaled columns keep
their values; the defining identity X' W'^T = X W^T (the emulated GEMM of the scaled parts against the FP64
product of the unscaled inputs, within the split bound), which a sign error on the weight side fails; and
on massive-activation inputs the calibrated split keeps near-FP32 accuracy where the plain row prescale
pushes the ordinary values beside a massive channel into FP16 subnormals."""
import numpy as np

import oracle
import workloads


def test_channel_exponents_by_hand():
    x = np.array([[1.0, 300.0, -0.5, 0.0, 512.0],
                  [2.0, -1000.0, 0.0, 0.0, -511.0]], np.float32)
    # column maxima 2, 1000 (ilogb 9), 0.5, 0 (all-zero), 512 (ilogb 9); T = 8
    assert oracle.channel_exponents(x, 8).tolist() == [0, -1, 0, 0, -1]
    assert oracle.channel_exponents(x, 9).tolist() == [0, 0, 0, 0, 0]
    assert oracle.channel_exponents(x, -3).tolist() == [-4, -12, -2, 0, -12]


def test_scaled_columns_land_below_the_threshold():
    x, idx = workloads.massive_channels(64, 512, seed=1)
    T = -12
    c = oracle.channel_exponents(x, T)
    xs = oracle.scale_columns(x, c, +1)
    m = np.abs(xs).max(0)
    assert np.all(m < 2.0 ** (T + 1))
    assert np.all(c[idx] < 0)                                     # the massive channels are the scaled ones
    plain = np.setdiff1d(np.arange(512), np.nonzero(c)[0])
    assert np.array_equal(xs[:, plain], x[:, plain])             # the others are untouched
    assert np.array_equal(oracle.scale_columns(xs, c, -1), x)    # exact both ways


def _emul_split(a, c, sign):
    hi, lo, e = oracle.split_f32(oracle.scale_columns(a, c, sign))
    return hi, lo, e


def _stress(M=64, K=1024, N=128, seed=3):
    x, idx = workloads.massive_channels(M, K, seed=seed)
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[: N // 2][:, idx] = 0.0  # the first half of the outputs never sees the massive channels
    return x, w, idx


def test_identity_and_sign():
    x, w, _ = _stress()
    c = oracle.channel_exponents(x, -12)
    ref = oracle.gemm_f64(x.astype(np.float64), w.astype(np.float64))
    absab = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    ah, al, ea = _emul_split(x, c, +1)
    bh, bl, eb = _emul_split(w, c, -1)
    ce, _ = oracle.gemm_emul(ah, al, ea, bh, bl, eb)
    assert np.all(np.abs(ce - ref) <= 4 * 2.0 ** -22 * absab)
    # the weight side scaled the wrong way round is caught
    bh2, bl2, eb2 = _emul_split(w, c, +1)
    ce2, _ = oracle.gemm_emul(ah, al, ea, bh2, bl2, eb2)
    assert np.max(np.abs(ce2 - ref) / (absab + 1e-300)) > 1e-2  # vs the 2^-20 bound above


def test_massive_channels_need_the_calibration():
    x, w, _ = _stress()
    ref = oracle.gemm_f64(x.astype(np.float64), w.astype(np.float64))
    half = slice(0, w.shape[0] // 2)  # outputs made of the ordinary values only
    rel = lambda ce: np.linalg.norm(ce[:, half] - ref[:, half]) / np.linalg.norm(ref[:, half])
    z = np.zeros(x.shape[1], np.int32)
    plain, _ = oracle.gemm_emul(*_emul_split(x, z, +1), *_emul_split(w, z, -1))
    c = oracle.channel_exponents(x, -12)
    calib, _ = oracle.gemm_emul(*_emul_split(x, c, +1), *_emul_split(w, c, -1))
    assert rel(plain) > 1e-4     # ordinary values beside a 1e5 channel fall into FP16 subnormals
    assert rel(calib) < 2e-7
