"""Pins of the oracle's 16-bit conversions (IEEE 754 round-to-nearest-even, gradual underflow).

These reduce to library routines: torch's CPU float32 -> float16 cast (hardware F16C conversion) and
float32 -> bfloat16 cast.  Every one of the 2^32 fp32 bit patterns is compared, so a wrong tie rule,
a missed subnormal or an off-by-one overflow threshold in the oracle fails here."""
import numpy as np
import pytest
import torch

import oracle


def test_hand_values():
    # values whose encodings follow from the binary16 / bfloat16 layouts by hand
    assert oracle.f16_bits(np.float32([1.0]))[0] == 0x3C00
    assert oracle.f16_bits(np.float32([65504.0]))[0] == 0x7BFF            # largest finite
    assert oracle.f16_bits(np.float32([65520.0]))[0] == 0x7C00            # halfway to 2^16: ties to even -> inf
    assert oracle.f16_bits(np.float32([65519.99]))[0] == 0x7BFF
    assert oracle.f16_bits(np.float32([2.0 ** -24]))[0] == 0x0001         # smallest subnormal
    assert oracle.f16_bits(np.float32([2.0 ** -25]))[0] == 0x0000         # tie with 0 -> even (0)
    assert oracle.f16_bits(np.float32([3 * 2.0 ** -25]))[0] == 0x0002     # tie 1.5 ulp -> 2 (even)
    assert oracle.f16_bits(np.float32([1 + 2.0 ** -11]))[0] == 0x3C00     # tie -> even mantissa
    assert oracle.f16_bits(np.float32([1 + 3 * 2.0 ** -11]))[0] == 0x3C02
    assert oracle.f16_bits(np.float32([-2.0]))[0] == 0xC000
    assert oracle.bf16_bits(np.float32([1.0]))[0] == 0x3F80
    assert oracle.bf16_bits(np.float32([1 + 2.0 ** -8]))[0] == 0x3F80     # tie -> even
    assert oracle.bf16_bits(np.float32([1 + 3 * 2.0 ** -8]))[0] == 0x3F82
    assert oracle.bf16_bits(np.float32([2.0 ** -133]))[0] == 0x0001       # smallest bf16 subnormal
    assert oracle.f16_value(0x7BFF) == 65504.0
    assert oracle.f16_value(0x0001) == 2.0 ** -24
    assert oracle.bf16_value(0x0001) == 2.0 ** -133
    assert oracle.bf16_value(0x7F7F) == (2 - 2.0 ** -7) * 2.0 ** 127


@pytest.mark.slow
def test_exhaustive_all_fp32_patterns():
    base = np.arange(1 << 24, dtype=np.uint32)
    u = np.empty(1 << 24, np.uint32)
    for c in range(256):
        np.add(base, np.uint32(c << 24), out=u)
        x = u.view(np.float32)
        xt = torch.from_numpy(x)
        nan = np.isnan(x)
        h = oracle.f16_bits(x)
        hr = xt.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(h[~nan], hr[~nan]), f"fp16 mismatch in chunk {c}"
        assert np.all((h[nan] & 0x7C00) == 0x7C00) and np.all((h[nan] & 0x03FF) != 0)
        b = oracle.bf16_bits(x)
        br = xt.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(b[~nan], br[~nan]), f"bf16 mismatch in chunk {c}"
        assert np.all((b[nan] & 0x7F80) == 0x7F80) and np.all((b[nan] & 0x007F) != 0)


def test_decode_all_16bit_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref16 = bits.view(np.float16).astype(np.float64)
    got16 = oracle.part_values(bits, oracle.F16)
    fin = np.isfinite(ref16)
    assert np.array_equal(got16[fin], ref16[fin])
    assert np.array_equal(np.isnan(got16), np.isnan(ref16))
    refb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    gotb = oracle.part_values(bits, oracle.BF16)
    fin = np.isfinite(refb)
    assert np.array_equal(gotb[fin], refb[fin])
    assert np.array_equal(np.isnan(gotb), np.isnan(refb))
