"""GPU parity of the paged INT16 decode (heal_attn_decode_paged).

Bar: normwise relative error <= 2e-6 against the oracle's FP64 attention on the dequantised values of each
sequence's gathered keys, and bit for bit against the contiguous decode of heal_attn_dual_fp16 on the same
keys (the same steps, splits and merge order run in both).  Page tables are shuffled, lengths ragged."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, dev, host, normwise

pytestmark = pytest.mark.gpu
TOL = 2e-6
D = 128


def _case(B, lens, Hq, Hkv, ps, seed):
    Lmax = max(max(lens), 1)
    q, qs = workloads.int16_cache_host(B, 1, Hq, D, seed=seed)
    k, ks = workloads.int16_cache_host(B, Lmax, Hkv, D, seed=seed + 1)
    v, vs = workloads.int16_cache_host(B, Lmax, Hkv, D, seed=seed + 2)
    P, tab = workloads.paged_layout(lens, ps, seed=seed + 3)
    kp = workloads.pages_from_contiguous(k, lens, tab, P, ps)
    vp = workloads.pages_from_contiguous(v, lens, tab, P, ps)
    ksp = workloads.pages_from_contiguous(ks, lens, tab, P, ps, fill=1.0)
    vsp = workloads.pages_from_contiguous(vs, lens, tab, P, ps, fill=1.0)
    return q[:, 0], qs[:, 0], kp, ksp, vp, vsp, tab


@pytest.mark.parametrize("B,lens,Hq,Hkv,ps,max_kv", [
    (3, [1, 77, 300], 8, 2, 32, None),
    (2, [0, 64], 4, 4, 64, None),           # an empty sequence: its row is 0
    (2, [33, 5000], 32, 8, 128, None),
    (1, [20000], 4, 1, 256, None),          # beyond 8192 keys
    (2, [100, 2100], 16, 2, 64, 6000),      # max_kv_len above every length: empty splits merge to nothing
    (1, [500], 8, 8, 32, 300),              # a length above max_kv_len is clamped to it
])
def test_paged_decode_vs_oracle(heal, B, lens, Hq, Hkv, ps, max_kv):
    banner(f"paged decode B={B} lens={lens} Hq={Hq} Hkv={Hkv} page={ps} max_kv_len={max_kv}")
    q, qs, kp, ksp, vp, vsp, tab = _case(B, lens, Hq, Hkv, ps, seed=31)
    mk = max(lens) if max_kv is None else max_kv
    need = -(-mk // ps)  # the table must have room for max_kv_len keys; the extra columns are never read
    if tab.shape[1] < need:
        tab = np.concatenate([tab, np.full((B, need - tab.shape[1]), -1, np.int32)], 1)
    out = heal.heal_attn_decode_paged(dev(q), dev(qs), dev(kp), dev(ksp), dev(vp), dev(vsp), dev(tab),
                                      dev(np.array(lens, np.int32)), mk)
    torch.cuda.synchronize()
    eff = np.minimum(np.array(lens), mk)
    want = oracle.attn_paged_i16_f64(q, qs, kp, ksp, vp, vsp, tab, eff)
    got = host(out)
    err = normwise(got, want)
    print(f"[paged] lens={lens} page={ps} normwise {err:.3e}")
    assert err <= TOL
    for b, n in enumerate(eff):
        if n == 0:
            assert np.all(got[b] == 0)


def test_paged_equals_contiguous_bitwise(heal):
    banner("paged decode == contiguous decode, 4 x 3000, GQA 16/4, page 64")
    B, L, Hq, Hkv, ps = 4, 3000, 16, 4, 64
    q, qs = workloads.int16_cache_host(B, 1, Hq, D, seed=41)
    k, ks = workloads.int16_cache_host(B, L, Hkv, D, seed=42)
    v, vs = workloads.int16_cache_host(B, L, Hkv, D, seed=43)
    lens = [L] * B
    P, tab = workloads.paged_layout(lens, ps, seed=44)
    pages = [workloads.pages_from_contiguous(t, lens, tab, P, ps, fill=f) for t, f in ((k, 0), (ks, 1.0), (v, 0),
                                                                                        (vs, 1.0))]
    paged = heal.heal_attn_decode_paged(dev(q[:, 0]), dev(qs[:, 0]), dev(pages[0]), dev(pages[1]), dev(pages[2]),
                                        dev(pages[3]), dev(tab), dev(np.array(lens, np.int32)), L)
    contig = heal.heal_attn_dual_fp16(dev(q), dev(qs), dev(k), dev(ks), dev(v), dev(vs), causal=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(paged).view(np.uint32), host(contig)[:, 0].view(np.uint32))


def test_paged_invalid_table_entries_stay_in_bounds(heal):
    banner("paged decode with out-of-range page ids (clamped in the kernel)")
    q, qs, kp, ksp, vp, vsp, tab = _case(2, [100, 300], 8, 2, 32, seed=51)
    tab = tab.copy()
    tab[0, 1] = -5
    tab[1, 3] = 10 ** 6
    out = heal.heal_attn_decode_paged(dev(q), dev(qs), dev(kp), dev(ksp), dev(vp), dev(vsp), dev(tab),
                                      dev(np.array([100, 300], np.int32)), 300)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


def test_paged_config_64x8192_equals_contiguous(heal):
    banner("paged decode 64 x 8192, GQA 32/8, page 64, shuffled pool == contiguous decode")
    B, L, Hq, Hkv, ps = 64, 8192, 32, 8, 64
    k, ks = workloads.int16_cache_device(B, L, Hkv, D, seed=3)
    v, vs = workloads.int16_cache_device(B, L, Hkv, D, seed=4)
    qh, qsh = workloads.int16_cache_host(B, 1, Hq, D, seed=5)
    q, qs = dev(qh), dev(qsh)
    npg = L // ps
    g = torch.Generator(device="cpu")
    g.manual_seed(6)
    perm = torch.randperm(B * npg + 5, generator=g).to("cuda")
    tab = perm[:B * npg].view(B, npg).to(torch.int32).contiguous()
    P = B * npg + 5

    def pool(t):
        p = torch.zeros((P, ps) + tuple(t.shape[2:]), dtype=t.dtype, device="cuda")
        p.index_copy_(0, tab.view(-1).long(), t.reshape((B * npg, ps) + tuple(t.shape[2:])))
        return p

    kp, ksp, vp, vsp = pool(k), pool(ks), pool(v), pool(vs)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    paged = heal.heal_attn_decode_paged(q[:, 0].contiguous(), qs[:, 0].contiguous(), kp, ksp, vp, vsp, tab, lens, L)
    contig = heal.heal_attn_dual_fp16(q, qs, k, ks, v, vs, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(paged.view(torch.int32), contig[:, 0].contiguous().view(torch.int32))
