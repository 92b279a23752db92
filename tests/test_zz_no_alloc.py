"""heal_attn_dual_fp16_noalloc, the entry point for callers that cannot allocate, against heal_attn_dual_fp16 with
a caller workspace: the same kernels, so the same output bits, on two decode calls in a row (the second smaller,
so it reuses scratch the first left behind), plus a prefill call (no scratch) and the FP64 oracle's bar."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, dev, host, normwise

pytestmark = pytest.mark.gpu


def _pair(heal, B, L, Hq, Hkv, Lq, seed, reading="byte"):
    q, qs = workloads.int16_cache_host(B, Lq, Hq, 128, seed=seed)
    k, ks = workloads.int16_cache_host(B, L, Hkv, 128, seed=seed + 1)
    v, vs = workloads.int16_cache_host(B, L, Hkv, 128, seed=seed + 2)
    t = [dev(a) for a in (q, qs, k, ks, v, vs)]
    ref_out = heal.heal_attn_dual_fp16(*t, causal=True, dual_split=reading)
    out = torch.full((B, Lq, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    heal.heal_attn_dual_fp16_noalloc(*t, out, causal=True, dual_split=reading)
    torch.cuda.synchronize()
    return (q, qs, k, ks, v, vs), host(ref_out), host(out)


@pytest.mark.parametrize("reading", ["byte", "float"])
def test_noalloc_equals_workspace_call(heal, reading):
    # first call: 16 sequences x 3000 keys, 32 / 8 heads (16 * 32 * 2 partials); second: smaller
    for (B, L, Hq, Hkv, seed) in ((16, 3000, 32, 8, 50), (3, 700, 8, 2, 60)):
        banner(f"noalloc decode B={B} L={L} Hq={Hq} Hkv={Hkv} {reading}")
        ins, want, got = _pair(heal, B, L, Hq, Hkv, 1, seed, reading)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        sel = [0, B - 1]
        ref = oracle.attn_i16_f64(*(a[sel] for a in ins), causal=True)
        err = normwise(got[sel], ref)
        print(f"[noalloc] decode {B}x{L} normwise {err:.3e}")
        assert err <= 2e-6
    banner("noalloc prefill (no scratch)")
    _, want, got = _pair(heal, 1, 200, 4, 2, 200, 70, reading)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_noalloc_refuses_oversize(heal):
    banner("noalloc refuses a decode over its scratch")
    q = torch.zeros((64, 1, 32, 128), dtype=torch.int16, device="cuda")
    qs = torch.zeros((64, 1, 32), dtype=torch.float32, device="cuda")
    # strides of a 20000-key cache over a small real buffer: refused on the host, nothing is launched
    k = torch.zeros((8, 128), dtype=torch.int16, device="cuda").as_strided((64, 20000, 8, 128),
                                                                          (0, 0, 128, 1))
    ks = torch.zeros((8,), dtype=torch.float32, device="cuda").as_strided((64, 20000, 8), (0, 0, 1))
    out = torch.zeros((64, 1, 32, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="WORKSPACE"):
        heal.heal_attn_dual_fp16_noalloc(q, qs, k, ks, k, ks, out, causal=True)
    torch.cuda.synchronize()
    assert bool((out == 0).all())
