"""GPU parity of the Dual-FP16 attention (prefill and decode) against the FP64 oracle on the dequantised
INT16 inputs.  Bar: normwise relative error <= 2e-6 over the checked rows; closed forms; decode equals
the last prefill row; run-to-run bit determinism."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import attn_row_errors, banner, dev, host, normwise

pytestmark = pytest.mark.gpu
TOL = 2e-6
# Every (b, i, h) row is also checked on its own, against sum_j p_j |v_j| (the row's scale without cancellation
# in the weighted sum), and the plain normwise error of the worst row is reported.  A row's error is not
# averaged with other rows': the FP32 accumulator that sums the three cross products of the INT16 halves in
# QK^T (hi lo, lo hi and lo lo, at scales 2^8 apart) rounds, and on the 1 x 4096 x 32 lognormal-scaled prefill
# the worst of 384 sampled rows measures 4.8e-6 while the whole tensor measures 9.1e-7.  The per-row bar is
# therefore 1e-5, five times the tensor bar.
ROW_TOL = 1e-5


def _rows(tag, got, q, qs, k, ks, v, vs, causal, ref, rows=None):
    wr, wc = attn_row_errors(got, q, qs, k, ks, v, vs, causal, ref, rows)
    print(f"[attn] {tag}: worst row normwise {wr:.3e}, worst row over sum p|v| {wc:.3e}")
    assert wc <= ROW_TOL


def _run(heal, q, qs, k, ks, v, vs, causal, scale=None):
    out = heal.heal_attn_dual_fp16(dev(q), dev(qs), dev(k), dev(ks), dev(v), dev(vs), causal=causal,
                                   softmax_scale=scale)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("B,Lq,Lkv,Hq,Hkv,causal", [
    (1, 300, 300, 4, 2, True), (2, 64, 64, 2, 2, False), (1, 77, 333, 3, 1, True), (1, 513, 513, 2, 1, True),
    (1, 5, 5, 1, 1, True), (1, 40, 17, 2, 2, True), (2, 33, 129, 4, 4, False)])
def test_prefill_small(heal, B, Lq, Lkv, Hq, Hkv, causal):
    banner(f"prefill B={B} Lq={Lq} Lkv={Lkv} Hq={Hq} Hkv={Hkv} causal={causal}")
    q, qs = workloads.int16_cache_host(B, Lq, Hq, 128, seed=11)
    k, ks = workloads.int16_cache_host(B, Lkv, Hkv, 128, seed=12)
    v, vs = workloads.int16_cache_host(B, Lkv, Hkv, 128, seed=13)
    o = _run(heal, q, qs, k, ks, v, vs, causal)
    ref = oracle.attn_i16_f64(q, qs, k, ks, v, vs, causal)
    err = normwise(o, ref)
    print(f"[attn] prefill {B},{Lq},{Lkv},{Hq},{Hkv},{causal} normwise {err:.3e}")
    assert err <= TOL
    _rows("prefill", o, q, qs, k, ks, v, vs, causal, ref)


def test_prefill_quantized_fp32_inputs(heal):
    banner("prefill from fp32 Q/K/V through the GPU quantiser")
    Q, K, V = workloads.qkv_fp32(1, 384, 4, 128, seed=2)
    qd, kd, vd = dev(Q[0]), dev(K[0]), dev(V[0])
    (q, qs), (k, ks), (v, vs) = (heal.heal_qkv_quant_i16(t) for t in (qd, kd, vd))
    out = heal.heal_attn_dual_fp16(q[None], qs[None], k[None], ks[None], v[None], vs[None], causal=True)
    torch.cuda.synchronize()
    oq, oqs = oracle.quant_i16(Q[0])
    ok_, oks = oracle.quant_i16(K[0])
    ov, ovs = oracle.quant_i16(V[0])
    ref = oracle.attn_i16_f64(oq[None], oqs[None], ok_[None], oks[None], ov[None], ovs[None], causal=True)
    err = normwise(host(out), ref)
    raw = oracle.attn_f64(Q, K, V, causal=True)
    qerr = normwise(host(out), raw)
    print(f"[attn] quantised prefill normwise {err:.3e} (vs raw fp32 inputs: {qerr:.3e})")
    assert err <= TOL


def test_closed_forms(heal):
    banner("attention closed forms")
    # one key with a power-of-two scale: O = s_v * v exactly
    q, qs = workloads.int16_cache_host(1, 4, 2, 128, seed=1)
    k, ks = workloads.int16_cache_host(1, 1, 2, 128, seed=2)
    v, _ = workloads.int16_cache_host(1, 1, 2, 128, seed=3)
    vs = np.full((1, 1, 2), 2.0 ** -13, np.float32)
    o = _run(heal, q, qs, k, ks, v, vs, causal=False)
    assert np.array_equal(o, np.broadcast_to(v.astype(np.float64) * 2.0 ** -13, o.shape).astype(np.float32))
    # identical value rows: O equals that row (decode and prefill)
    for Lq in (1, 70):
        k, ks = workloads.int16_cache_host(1, 200, 1, 128, seed=4)
        v1, _ = workloads.int16_cache_host(1, 1, 1, 128, seed=5)
        v = np.repeat(v1, 200, axis=1)
        vs = np.full((1, 200, 1), 3.0e-4, np.float32)
        q, qs = workloads.int16_cache_host(1, Lq, 4, 128, seed=6)
        o = _run(heal, q, qs, k, ks, v, vs, causal=True)
        want = (v1[0, 0, 0].astype(np.float64) * np.float64(np.float32(3.0e-4)))
        assert normwise(o.reshape(-1, 128), np.broadcast_to(want, (Lq * 4, 128))) <= 1e-6


def test_decode_matches_last_prefill_row(heal):
    banner("decode == last row of prefill")
    B, L, Hq, Hkv = 2, 1500, 8, 2
    q, qs = workloads.int16_cache_host(B, L, Hq, 128, seed=21)
    k, ks = workloads.int16_cache_host(B, L, Hkv, 128, seed=22)
    v, vs = workloads.int16_cache_host(B, L, Hkv, 128, seed=23)
    full = _run(heal, q, qs, k, ks, v, vs, causal=True)
    dec = _run(heal, q[:, -1:], qs[:, -1:], k, ks, v, vs, causal=True)
    ref = oracle.attn_i16_f64(q[:, -1:], qs[:, -1:], k, ks, v, vs, causal=True)
    e_dec, e_full = normwise(dec, ref), normwise(full[:, -1:], ref)
    print(f"[attn] decode {e_dec:.3e}, last prefill row {e_full:.3e}")
    assert e_dec <= TOL and e_full <= TOL
    assert normwise(dec, full[:, -1:]) <= 2 * TOL


@pytest.mark.parametrize("B,L,Hq,Hkv", [(3, 1000, 32, 8), (1, 1, 4, 4), (2, 4097, 16, 1), (1, 33, 8, 8),
                                        (2, 700, 32, 1)])  # 32 query heads per kv head: the prefill kernel
def test_decode_small(heal, B, L, Hq, Hkv):
    banner(f"decode B={B} L={L} Hq={Hq} Hkv={Hkv}")
    q, qs = workloads.int16_cache_host(B, 1, Hq, 128, seed=31)
    k, ks = workloads.int16_cache_host(B, L, Hkv, 128, seed=32)
    v, vs = workloads.int16_cache_host(B, L, Hkv, 128, seed=33)
    o = _run(heal, q, qs, k, ks, v, vs, causal=True)
    ref = oracle.attn_i16_f64(q, qs, k, ks, v, vs, causal=True)
    err = normwise(o, ref)
    print(f"[attn] decode {B},{L},{Hq},{Hkv} normwise {err:.3e}")
    assert err <= TOL
    _rows("decode", o, q, qs, k, ks, v, vs, True, ref)


# The decode plan: 512 keys per wavefront, halved (down to 32) while the grid would hold fewer than 512
# workgroups; the workspace holds one partial per (batch, query head, chunk of 4 wavefronts' keys), so its
# size shows the plan taken.  Each case has a ragged last chunk.
@pytest.mark.parametrize("B,L,Hq,Hkv,kpw", [(64, 2500, 32, 8, 512), (24, 3000, 32, 8, 256),
                                            (16, 3000, 32, 8, 128), (4, 5000, 32, 8, 64), (1, 575, 32, 8, 32)])
def test_decode_plans(heal, B, L, Hq, Hkv, kpw):
    banner(f"decode plan B={B} L={L} Hq={Hq} Hkv={Hkv}, {kpw} keys per wavefront")
    q, qs = workloads.int16_cache_host(B, 1, Hq, 128, seed=34)
    k, ks = workloads.int16_cache_host(B, L, Hkv, 128, seed=35)
    v, vs = workloads.int16_cache_host(B, L, Hkv, 128, seed=36)
    args = [dev(t) for t in (q, qs, k, ks, v, vs)]
    out = torch.empty((B, 1, Hq, 128), dtype=torch.float32, device="cuda")
    need = heal.heal_attn_workspace_bytes(heal.make_attn_args(*args, out))
    assert need == B * Hq * -(-L // (4 * kpw)) * (4 + 128) * 4
    o1 = heal.heal_attn_dual_fp16(*args, causal=True)
    o2 = heal.heal_attn_dual_fp16(*args, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
    sel = sorted({0, B // 2, B - 1})
    ref = oracle.attn_i16_f64(q[sel], qs[sel], k[sel], ks[sel], v[sel], vs[sel], causal=True)
    err = normwise(host(o1)[sel], ref)
    print(f"[attn] decode plan {B},{L} kpw {kpw} normwise {err:.3e}")
    assert err <= TOL
    _rows("decode plan", host(o1)[sel], q[sel], qs[sel], k[sel], ks[sel], v[sel], vs[sel], True, ref)


def test_prefill_config_sampled_and_deterministic(heal):
    banner("prefill 1x4096x32x128 causal, sampled rows")
    B, L, H = 1, 4096, 32
    Q, K, V = workloads.qkv_fp32(B, L, H, 128, seed=2)
    qd, kd, vd = dev(Q[0]), dev(K[0]), dev(V[0])
    (q, qs), (k, ks), (v, vs) = (heal.heal_qkv_quant_i16(t) for t in (qd, kd, vd))
    args = (q[None], qs[None], k[None], ks[None], v[None], vs[None])
    o1 = heal.heal_attn_dual_fp16(*args, causal=True)
    o2 = heal.heal_attn_dual_fp16(*args, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
    oq, oqs = oracle.quant_i16(Q[0])
    ok_, oks = oracle.quant_i16(K[0])
    ov, ovs = oracle.quant_i16(V[0])
    assert np.array_equal(host(q), oq) and np.array_equal(host(k), ok_) and np.array_equal(host(v), ov)
    rng = np.random.default_rng(0)
    rows = np.stack([np.zeros(384, np.int64), rng.integers(0, L, 384), rng.integers(0, H, 384)], 1)
    rows[:8, 1] = [0, 1, 255, 256, 4094, 4095, 63, 64]
    ref = oracle.attn_i16_f64(oq[None], oqs[None], ok_[None], oks[None], ov[None], ovs[None], True, rows=rows)
    got = host(o1)[rows[:, 0], rows[:, 1], rows[:, 2]]
    err = normwise(got, ref)
    print(f"[attn] prefill 4096 sampled normwise {err:.3e}")
    assert err <= TOL
    _rows("prefill 4096 sampled", got, oq[None], oqs[None], ok_[None], oks[None], ov[None], ovs[None], True, ref,
          rows)


def test_decode_config_sampled(heal):
    banner("decode 64x8192 GQA 32/8, sampled heads")
    B, L, Hq, Hkv = 64, 8192, 32, 8
    k, ks = workloads.int16_cache_device(B, L, Hkv, 128, seed=3)
    v, vs = workloads.int16_cache_device(B, L, Hkv, 128, seed=4)
    qh, qsh = workloads.int16_cache_host(B, 1, Hq, 128, seed=5)
    q, qs = dev(qh), dev(qsh)
    out = heal.heal_attn_dual_fp16(q, qs, k, ks, v, vs, causal=True)
    torch.cuda.synchronize()
    o = host(out)
    errs = []
    for b in (0, 17, 63):
        kb, ksb, vb, vsb = (host(t[b:b + 1]) for t in (k, ks, v, vs))
        ref = oracle.attn_i16_f64(qh[b:b + 1], qsh[b:b + 1], kb, ksb, vb, vsb, causal=True)
        errs.append(normwise(o[b:b + 1], ref))
        _rows(f"decode 64x8192 batch {b}", o[b:b + 1], qh[b:b + 1], qsh[b:b + 1], kb, ksb, vb, vsb, True, ref)
    print(f"[attn] decode 64x8192 sampled normwise {max(errs):.3e}")
    assert max(errs) <= TOL


def _all_codes(rng, shape):
    """int16 codes [.., L, H, D] in which every one of the 65,536 values appears (the leading tokens hold
    permutations of the whole range), followed by two tokens whose codes are all -32768 and all +32767."""
    B, L, H, D = shape
    n = B * L * H * D
    assert n % 65536 == 0
    allv = np.arange(-32768, 32768, dtype=np.int32).astype(np.int16)
    body = np.concatenate([rng.permutation(allv) for _ in range(n // 65536)]).reshape(B, L, H, D)
    ends = np.empty((B, 2, H, D), np.int16)
    ends[:, 0] = -32768
    ends[:, 1] = 32767
    return np.concatenate([body, ends], axis=1)


def _scales(rng, B, L, H):
    return np.broadcast_to(np.exp(rng.standard_normal((B, L, 1))) / 32768.0, (B, L, H)).astype(np.float32).copy()


@pytest.mark.parametrize("reading", ["byte", "shift10", "float"])
def test_full_int16_range(heal, reading):
    """Q, K and V codes covering every INT16 value, -32768 included (which the quantiser never writes but the
    interface accepts), and constant rows at both ends of the range, through the in-register unpack of each
    reading of the pair: causal prefill, and decode with grouped query heads."""
    banner(f"attention over every INT16 code, {reading} reading")
    rng = np.random.default_rng(40)
    q, k, v = (_all_codes(rng, (1, 512, 1, 128)) for _ in range(3))
    qs, ks, vs = (_scales(rng, 1, 514, 1) for _ in range(3))
    out = heal.heal_attn_dual_fp16(dev(q), dev(qs), dev(k), dev(ks), dev(v), dev(vs), causal=True,
                                   dual_split=reading)
    torch.cuda.synchronize()
    ref = oracle.attn_i16_f64(q, qs, k, ks, v, vs, causal=True)
    err = normwise(host(out), ref)
    print(f"[attn] full-range prefill ({reading}) normwise {err:.3e}")
    assert err <= TOL
    _rows(f"full-range prefill ({reading})", host(out), q, qs, k, ks, v, vs, True, ref)
    # decode: 2 sequences of 514 keys, 8 query heads over 2 key/value heads
    k, v = (_all_codes(rng, (2, 512, 2, 128)) for _ in range(2))
    ks, vs = (_scales(rng, 2, 514, 2) for _ in range(2))
    qd = rng.integers(-32768, 32768, (2, 1, 8, 128)).astype(np.int16)
    qd[0, 0, 0] = -32768
    qd[1, 0, 7] = 32767
    qds = _scales(rng, 2, 1, 8)
    out = heal.heal_attn_dual_fp16(dev(qd), dev(qds), dev(k), dev(ks), dev(v), dev(vs), causal=True,
                                   dual_split=reading)
    torch.cuda.synchronize()
    ref = oracle.attn_i16_f64(qd, qds, k, ks, v, vs, causal=True)
    err = normwise(host(out), ref)
    print(f"[attn] full-range decode ({reading}) normwise {err:.3e}")
    assert err <= TOL
    _rows(f"full-range decode ({reading})", host(out), qd, qds, k, ks, v, vs, True, ref)
