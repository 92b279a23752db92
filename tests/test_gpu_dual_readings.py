"""GPU parity of the three readings of the Dual-FP16 pair ([TS 2A Mechanism]: an INT16 value becomes two
exact FP16 values): the byte split (the default), the split at bit 10, and the float-float pair.

Bar: the standalone unpack bit for bit against the oracle over every INT16 value; attention (prefill,
decode, paged decode) under each reading at normwise relative error <= 2e-6 against the oracle's FP64
attention on the dequantised inputs, the same bar as the default reading; the paged decode bit for bit
against the contiguous decode of the same reading."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, bits, dev, host, normwise

pytestmark = pytest.mark.gpu
TOL = 2e-6
READINGS = ("byte", "shift10", "float")


@pytest.mark.parametrize("reading", READINGS)
def test_unpack_exhaustive(heal, reading):
    banner(f"unpack i16 all 65536 values, reading {reading}")
    q = np.arange(-32768, 32768, dtype=np.int32).astype(np.int16).reshape(256, 256)
    hi, lo = heal.heal_unpack_i16(dev(q), reading)
    torch.cuda.synchronize()
    ohi, olo = oracle.unpack_i16(q, reading)
    assert np.array_equal(bits(hi), ohi) and np.array_equal(bits(lo), olo)
    # ragged columns and a row stride that is not a multiple of 8 (element-wise path)
    qd = dev(q)[:7, 3:16]
    hi, lo = heal.heal_unpack_i16(qd, reading)
    torch.cuda.synchronize()
    ohi, olo = oracle.unpack_i16(q[:7, 3:16], reading)
    assert np.array_equal(bits(hi), ohi) and np.array_equal(bits(lo), olo)


def test_unpack_byte_equals_split(heal):
    banner("unpack byte reading == heal_split(int16)")
    q = workloads.int16_cache_host(1, 300, 2, 128, seed=5)[0].reshape(600, 128)
    h1, l1 = heal.heal_unpack_i16(dev(q), "byte")
    h2, l2, _ = heal.heal_split(dev(q))
    torch.cuda.synchronize()
    assert np.array_equal(bits(h1), bits(h2)) and np.array_equal(bits(l1), bits(l2))


def _attn(heal, reading, q, qs, k, ks, v, vs, causal):
    out = heal.heal_attn_dual_fp16(dev(q), dev(qs), dev(k), dev(ks), dev(v), dev(vs), causal=causal,
                                   dual_split=reading)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("reading", READINGS)
@pytest.mark.parametrize("B,Lq,Lkv,Hq,Hkv,causal", [
    (1, 300, 300, 4, 2, True), (2, 33, 129, 4, 4, False), (1, 77, 333, 3, 1, True), (1, 5, 5, 1, 1, True)])
def test_prefill(heal, reading, B, Lq, Lkv, Hq, Hkv, causal):
    banner(f"prefill reading {reading} B={B} Lq={Lq} Lkv={Lkv} Hq={Hq} Hkv={Hkv} causal={causal}")
    q, qs = workloads.int16_cache_host(B, Lq, Hq, 128, seed=11)
    k, ks = workloads.int16_cache_host(B, Lkv, Hkv, 128, seed=12)
    v, vs = workloads.int16_cache_host(B, Lkv, Hkv, 128, seed=13)
    o = _attn(heal, reading, q, qs, k, ks, v, vs, causal)
    err = normwise(o, oracle.attn_i16_f64(q, qs, k, ks, v, vs, causal))
    print(f"[dual] prefill {reading} {B},{Lq},{Lkv},{Hq},{Hkv},{causal} normwise {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("reading", READINGS)
@pytest.mark.parametrize("B,L,Hq,Hkv", [(3, 1000, 32, 8), (1, 1, 4, 4), (2, 4097, 16, 1), (1, 300, 24, 1)])
def test_decode(heal, reading, B, L, Hq, Hkv):
    banner(f"decode reading {reading} B={B} L={L} Hq={Hq} Hkv={Hkv}")
    q, qs = workloads.int16_cache_host(B, 1, Hq, 128, seed=31)
    k, ks = workloads.int16_cache_host(B, L, Hkv, 128, seed=32)
    v, vs = workloads.int16_cache_host(B, L, Hkv, 128, seed=33)
    o = _attn(heal, reading, q, qs, k, ks, v, vs, True)
    err = normwise(o, oracle.attn_i16_f64(q, qs, k, ks, v, vs, True))
    print(f"[dual] decode {reading} {B},{L},{Hq},{Hkv} normwise {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("reading", READINGS)
def test_paged_matches_oracle_and_contiguous(heal, reading):
    banner(f"paged decode reading {reading}")
    lens, Hq, Hkv, ps = [77, 3000], 16, 4, 64
    B, Lmax = len(lens), max(lens)
    q, qs = workloads.int16_cache_host(B, 1, Hq, 128, seed=41)
    k, ks = workloads.int16_cache_host(B, Lmax, Hkv, 128, seed=42)
    v, vs = workloads.int16_cache_host(B, Lmax, Hkv, 128, seed=43)
    P, tab = workloads.paged_layout(lens, ps, seed=44)
    kp = workloads.pages_from_contiguous(k, lens, tab, P, ps)
    vp = workloads.pages_from_contiguous(v, lens, tab, P, ps)
    ksp = workloads.pages_from_contiguous(ks, lens, tab, P, ps, fill=1.0)
    vsp = workloads.pages_from_contiguous(vs, lens, tab, P, ps, fill=1.0)
    out = heal.heal_attn_decode_paged(dev(q[:, 0]), dev(qs[:, 0]), dev(kp), dev(ksp), dev(vp), dev(vsp),
                                      dev(tab), dev(np.array(lens, np.int32)), Lmax, dual_split=reading)
    torch.cuda.synchronize()
    got = host(out)
    want = oracle.attn_paged_i16_f64(q[:, 0], qs[:, 0], kp, ksp, vp, vsp, tab, np.array(lens))
    err = normwise(got, want)
    print(f"[dual] paged {reading} normwise {err:.3e}")
    assert err <= TOL
    # the same keys through the contiguous decode of the same reading: bit for bit
    for b, n in enumerate(lens):
        o = heal.heal_attn_dual_fp16(dev(q[b:b + 1]), dev(qs[b:b + 1]), dev(k[b:b + 1, :n]), dev(ks[b:b + 1, :n]),
                                     dev(v[b:b + 1, :n]), dev(vs[b:b + 1, :n]), causal=True, dual_split=reading)
        torch.cuda.synchronize()
        assert np.array_equal(host(o)[0, 0].view(np.uint32), got[b].view(np.uint32))


@pytest.mark.parametrize("reading", ("shift10", "float"))
def test_prefill_config_sampled(heal, reading):
    banner(f"prefill 1x4096x32x128 causal, reading {reading}, sampled rows")
    B, L, H = 1, 4096, 32
    Q, K, V = workloads.qkv_fp32(B, L, H, 128, seed=2)
    (q, qs), (k, ks), (v, vs) = (heal.heal_qkv_quant_i16(dev(t[0])) for t in (Q, K, V))
    out = heal.heal_attn_dual_fp16(q[None], qs[None], k[None], ks[None], v[None], vs[None], causal=True,
                                   dual_split=reading)
    torch.cuda.synchronize()
    oq, oqs = oracle.quant_i16(Q[0])
    ok_, oks = oracle.quant_i16(K[0])
    ov, ovs = oracle.quant_i16(V[0])
    rng = np.random.default_rng(0)
    rows = np.stack([np.zeros(256, np.int64), rng.integers(0, L, 256), rng.integers(0, H, 256)], 1)
    rows[:6, 1] = [0, 1, 255, 256, 4094, 4095]
    ref = oracle.attn_i16_f64(oq[None], oqs[None], ok_[None], oks[None], ov[None], ovs[None], True, rows=rows)
    got = host(out)[rows[:, 0], rows[:, 1], rows[:, 2]]
    err = normwise(got, ref)
    print(f"[dual] prefill 4096 {reading} sampled normwise {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("reading", ("shift10", "float"))
def test_decode_config_sampled(heal, reading):
    banner(f"decode 64x8192 GQA 32/8, reading {reading}, sampled batches")
    B, L, Hq, Hkv = 64, 8192, 32, 8
    k, ks = workloads.int16_cache_device(B, L, Hkv, 128, seed=3)
    v, vs = workloads.int16_cache_device(B, L, Hkv, 128, seed=4)
    qh, qsh = workloads.int16_cache_host(B, 1, Hq, 128, seed=5)
    out = heal.heal_attn_dual_fp16(dev(qh), dev(qsh), k, ks, v, vs, causal=True, dual_split=reading)
    torch.cuda.synchronize()
    o = host(out)
    errs = []
    for b in (0, 63):
        kb, ksb, vb, vsb = (host(t[b:b + 1]) for t in (k, ks, v, vs))
        errs.append(normwise(o[b:b + 1], oracle.attn_i16_f64(qh[b:b + 1], qsh[b:b + 1], kb, ksb, vb, vsb, True)))
    print(f"[dual] decode 64x8192 {reading} sampled normwise {max(errs):.3e}")
    assert max(errs) <= TOL
