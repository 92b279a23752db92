"""Pins of the oracle's INT16 quantisation of Q/K/V ([TS 2A Solution]; [TS] = gist.science explainer
"Demystifying Numerical Instability in LLM Inference ... with HEAL", Technical Summary).

Pins: hand-derived rows with power-of-two scales (tests/golden) that fix ties-to-even and the clamp; the
error bound |x - s q| <= s (1/2 + 2^-9) of one IEEE division and one rounding; max|q| = 32767 on every
nonzero row; all-zero rows; independence of rows."""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_power_of_two_scales():
    for line in open(os.path.join(GOLDEN, "quant_i16_cases.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        f = line.split()
        k = int(f[0])
        xs = [float(v) for v in f[1::2]]
        qs = [int(v) for v in f[2::2]]
        row = np.zeros((1, 1, 1 + len(xs)), np.float32)
        row[0, 0, 0] = 32767.0 * 2.0 ** k
        row[0, 0, 1:] = np.array(xs) * 2.0 ** k
        q, s = oracle.quant_i16(row)
        assert s[0, 0] == np.float32(2.0 ** k)
        assert q[0, 0, 0] == 32767
        assert list(q[0, 0, 1:]) == qs, line


def test_bound_and_extremes():
    import workloads

    Q, _, _ = workloads.qkv_fp32(1, 64, 8, 128, seed=9)
    x = Q[0]
    x[3, 2, :] = 0.0
    x[4, 1, :] = -x[4, 1, :]
    x[5, 0, 7] = 1e-40  # subnormal alone in a row
    x[5, 0, :7] = 0.0
    x[5, 0, 8:] = 0.0
    q, s = oracle.quant_i16(x)
    xd = x.astype(np.float64)
    qd = q.astype(np.float64)
    sd = s.astype(np.float64)[..., None]
    nz = np.abs(x).max(-1) > 0
    normal = (s >= np.float32(2.0 ** -126))[..., None] | (xd == 0)
    err = np.abs(xd - sd * qd)
    # the bound of one IEEE division and one rounding holds while s is a normal fp32 number
    assert np.all((err <= sd * (0.5 + 2.0 ** -9)) | ~normal)
    # a row whose max is below 32767 * 2^-126 gets a subnormal scale: q still saturates at the max
    assert q[5, 0, 7] == 32767 and s[5, 0] > 0
    assert np.all(np.abs(q).max(-1)[nz] == 32767)
    assert np.all(q[3, 2] == 0) and s[3, 2] == 0
    assert np.array_equal(q[4, 1], -oracle.quant_i16(-x[4:5, 1:2])[0][0, 0])
    assert np.all(q >= -32767)


def test_rows_are_independent_and_scale_invariant():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 4, 128)).astype(np.float32)
    q1, s1 = oracle.quant_i16(x)
    # scaling a row by a power of two scales s by the same power and leaves q unchanged
    x2 = x.copy()
    x2[2, 3] *= np.float32(2.0 ** 20)
    q2, s2 = oracle.quant_i16(x2)
    assert np.array_equal(q1, q2)
    assert s2[2, 3] == s1[2, 3] * np.float32(2.0 ** 20)
    # a permutation of tokens permutes outputs
    perm = rng.permutation(16)
    q3, s3 = oracle.quant_i16(x[perm])
    assert np.array_equal(q3, q1[perm]) and np.array_equal(s3, s1[perm])
