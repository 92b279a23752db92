"""Pins of the oracle's split (the compensated GEMM's operand decomposition) and of the Dual-FP16 unpack.

Split: [TS 2B Mechanism], a 16-bit leading part plus the 16-bit remainder it leaves, with the exact power-of-two
row prescale standing for [TS 2B Overflow Handling].  Dual-FP16: [TS 2A Mechanism].  ([TS] is the
gist.science explainer "Demystifying Numerical Instability in LLM Inference ... with HEAL", Technical
Summary.)  Pins: hand-derived cases (tests/golden), invariants that hold for every input (property
tests), exhaustive enumeration of the 65,536 INT16 values."""
import math
import os
from fractions import Fraction

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ulp16(v):
    """spacing of the binary16 grid at |v| (subnormal spacing below 2^-14)"""
    if v == 0:
        return 2.0 ** -24
    return 2.0 ** (max(math.frexp(abs(v))[1] - 1, -14) - 10)


def test_golden_hand_cases():
    for line in open(os.path.join(GOLDEN, "split_f16_cases.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        xs, es, his, los = line.split()
        x = np.float32(float(xs))
        hi, lo, e = oracle.split_f32(np.array([[x]], np.float32))
        assert e[0] == int(es), line
        assert oracle.f16_value(hi[0, 0]) == float(his), line
        assert oracle.f16_value(lo[0, 0]) == float(los), line


def _check_row(row: np.ndarray):
    hi, lo, e = oracle.split_f32(row[None, :])
    amax = float(np.max(np.abs(row)))
    if amax == 0:
        assert e[0] == 0
    else:
        assert 2.0 ** 14 <= amax * 2.0 ** int(e[0]) < 2.0 ** 15
        assert -113 <= e[0] <= 163
    hv = oracle.part_values(hi[0], oracle.F16)
    lv = oracle.part_values(lo[0], oracle.F16)
    for c in range(row.size):
        xs = Fraction(float(np.float32(float(row[c]) * 2.0 ** int(e[0]))))  # x' as stored in fp32
        h, l = Fraction(hv[c]), Fraction(lv[c])
        assert abs(hv[c]) <= 2.0 ** 15
        # hi is the nearest fp16 to x'
        assert abs(xs - h) <= Fraction(_ulp16(float(h))) / 2 or abs(xs - h) <= Fraction(_ulp16(float(xs))) / 2
        # hi + lo reconstructs x' within half a unit of lo's own fp16 grid (the residual's rounding)
        assert abs(xs - (h + l)) <= Fraction(_ulp16(float(xs - h))) / 2
        # x' itself is x scaled exactly unless it fell below the fp32 normal range
        if abs(float(row[c])) * 2.0 ** int(e[0]) >= 2.0 ** -126 or row[c] == 0:
            assert xs == Fraction(float(row[c])) * Fraction(2) ** int(e[0])


@settings(max_examples=300, deadline=None)
@given(st.lists(st.floats(allow_nan=False, allow_infinity=False, width=32),
                min_size=1, max_size=12))
def test_split_invariants_property(vals):
    _check_row(np.array(vals, np.float32))


def test_split_invariants_wide_rows():
    rng = np.random.default_rng(11)
    for scale in (1e-30, 1e-5, 1.0, 3e4, 1e30):
        row = (rng.standard_normal(64) * scale).astype(np.float32)
        row[5] = 0.0
        _check_row(row)
    _check_row(np.zeros(7, np.float32))


def test_split_exact_when_22_bits():
    # an fp32 value with at most 22 significant bits below the row maximum's leading bit is reproduced exactly
    rng = np.random.default_rng(5)
    m = rng.integers(-(1 << 21), 1 << 21, size=256)
    x = (m.astype(np.float64) * 2.0 ** -20).astype(np.float32)
    x[0] = np.float32(2.0)  # row max in [2, 4): e = 13, x' = x * 2^13 has its grid at 2^-7
    hi, lo, e = oracle.split_f32(x[None, :])
    rec = oracle.part_values(hi[0], oracle.F16) + oracle.part_values(lo[0], oracle.F16)
    assert np.array_equal(rec, x.astype(np.float64) * 2.0 ** int(e[0]))


def test_split_binade_bruteforce():
    # every fp32 value in [1, 2) with a stride, in a row whose max is 1.999..: hi + lo == x' exactly
    # (x' has 24 bits; hi takes 11, the residual needs at most 13 and fits fp16's 11 + subnormal room? no:
    # the residual is rounded, so check the half-ulp bound instead, and exactness for 22-bit inputs)
    u = np.arange(0x3F800000, 0x40000000, 97, dtype=np.uint32)
    x = u.view(np.float32)
    for chunk in np.array_split(x, 64):
        row = np.concatenate([chunk, np.float32([1.9999999])])
        _check_row_fast(row)


def _check_row_fast(row):
    hi, lo, e = oracle.split_f32(row[None, :])
    xs = row.astype(np.float64) * 2.0 ** int(e[0])
    h = oracle.part_values(hi[0], oracle.F16)
    l = oracle.part_values(lo[0], oracle.F16)
    r = xs - h  # exact in double
    spacing_lo = np.array([_ulp16(v) for v in r])
    assert np.all(np.abs(xs - (h + l)) <= spacing_lo / 2)
    assert np.all(np.abs(r) <= np.array([_ulp16(v) for v in xs]) / 2)


def test_split_no_prescale_and_bf16():
    x = np.float32([[1.0 + 2.0 ** -9, -3.0, 0.0]])
    hi, lo, e = oracle.split_f32(x, part=oracle.BF16, prescale=False)
    assert list(e) == [0]
    h = oracle.part_values(hi[0], oracle.BF16)
    l = oracle.part_values(lo[0], oracle.BF16)
    assert h[0] == 1.0 and l[0] == 2.0 ** -9  # bf16 keeps 8 bits: hi = 1, residual exact in bf16
    assert h[1] == -3.0 and l[1] == 0.0
    hi, lo, e = oracle.split_f32(np.float32([[1e6]]), prescale=False)
    assert oracle.f16_value(hi[0, 0]) == math.inf  # unscaled FP16 overflows: why the prescale exists


def test_split_bf16_weights_exact_in_f16():
    # bf16 N(0, 0.02) weights: after the per-row prescale every value is exact in fp16 (8 <= 11 bits and no
    # value falls below fp16's subnormal grid within 2^-24 * 2^14 of the row max range that matters)
    import workloads

    W = workloads.llama_weights_bf16(64, 512, seed=3)
    hi, lo, e = oracle.split_bf16(W, residual=True)
    wv = oracle.part_values(W, oracle.BF16)
    hv = oracle.part_values(hi, oracle.F16)
    lv = oracle.part_values(lo, oracle.F16)
    scaled = wv * np.exp2(e.astype(np.float64))[:, None]
    small = np.abs(scaled) < 2.0 ** -14 * 2 ** 7  # values with fewer than 8 bits of fp16 room
    assert np.array_equal(hv[~small], scaled[~small])
    assert np.all(lv[~small] == 0)


def test_dual_fp16_exhaustive():
    q = np.arange(-32768, 32768, dtype=np.int32).astype(np.int16)
    hi, lo = oracle.split_i16(q[None, :])
    h = oracle.part_values(hi[0], oracle.F16)
    l = oracle.part_values(lo[0], oracle.F16)
    assert np.all(h == np.floor(q / 256.0))
    assert np.all((l >= 0) & (l <= 255))
    assert np.array_equal(256 * h + l, q.astype(np.float64))
    # both halves are integers of at most 8 bits: exact in fp16 (re-encoding reproduces the bit pattern)
    assert np.array_equal(oracle.f16_bits(h.astype(np.float32)), hi[0])
    assert np.array_equal(oracle.f16_bits(l.astype(np.float32)), lo[0])
    # exactness of FP32 partial sums over head_dim 128 for each product class (byte split)
    assert 128 * 128 * 128 < 2 ** 24 and 128 * 128 * 255 * 2 < 2 ** 24 and 128 * 255 * 255 < 2 ** 24


def test_dual_readings_golden():
    """Hand-derived pairs of all three readings of the Dual-FP16 pair ([TS 2A Mechanism]), including the
    ties of the float reading (2049 -> 2048, 2051 -> 2052) and both ends of the INT16 range."""
    cases = [list(map(int, l.split())) for l in open(os.path.join(GOLDEN, "dual_split_cases.txt"))
             if l.strip() and not l.startswith("#")]
    q = np.array([[c[0] for c in cases]], np.int16)
    for col, reading in ((1, "byte"), (3, "shift10"), (5, "float")):
        hi, lo = oracle.unpack_i16(q, reading)
        h = oracle.part_values(hi[0], oracle.F16)
        l = oracle.part_values(lo[0], oracle.F16)
        assert np.array_equal(h, [c[col] for c in cases]), reading
        assert np.array_equal(l, [c[col + 1] for c in cases]), reading


def test_dual_readings_exhaustive():
    """Every INT16 value under each reading: closed forms by integer arithmetic, numpy's own binary16
    rounding for the float reading, exact reconstruction, and FP16 exactness of every half."""
    q = np.arange(-32768, 32768, dtype=np.int32).astype(np.int16)
    qi = q.astype(np.int64)
    out = {}
    for reading in ("byte", "shift10", "float"):
        hi, lo = oracle.unpack_i16(q[None, :], reading)
        h = oracle.part_values(hi[0], oracle.F16)
        l = oracle.part_values(lo[0], oracle.F16)
        assert np.array_equal(oracle.f16_bits(h.astype(np.float32)), hi[0])  # exact in fp16
        assert np.array_equal(oracle.f16_bits(l.astype(np.float32)), lo[0])
        out[reading] = (h, l)
    h, l = out["byte"]
    assert np.array_equal(h, qi // 256) and np.array_equal(l, qi % 256)
    assert np.array_equal(256 * h + l, qi)
    bh, bl = oracle.split_i16(q[None, :])  # the default reading is the byte split
    assert np.array_equal(oracle.part_values(bh[0], oracle.F16), h)
    h, l = out["shift10"]
    assert np.array_equal(h, qi // 1024) and np.array_equal(l, qi % 1024)
    assert np.all((h >= -32) & (h <= 31)) and np.all((l >= 0) & (l <= 1023))
    assert np.array_equal(1024 * h + l, qi)
    h, l = out["float"]
    assert np.array_equal(h, q.astype(np.float16).astype(np.float64))  # numpy: round to nearest even
    assert np.array_equal(h + l / 1024.0, qi.astype(np.float64))
    assert np.all(np.abs(l) <= 16 * 1024)
    assert np.all(l[np.abs(qi) <= 2048] == 0)
    # FP32 exactness of the attention's accumulators at head_dim 128 (integer readings): shift-10 hi.hi
    # partial sums are multiples of 2^20 with |sum hi hi'| <= 128 * 32 * 32 = 2^17; the byte split's are
    # multiples of 2^16 with |sum| <= 128 * 128 * 128 = 2^21
    assert 128 * 32 * 32 <= 2 ** 17 and 128 * 128 * 128 <= 2 ** 21
