"""Pins of the oracle's attention (FP64 definition, graded on dequantised INT16 inputs; [TS 2A];
[TS] = gist.science explainer "Demystifying Numerical Instability in LLM Inference ... with HEAL",
Technical Summary).

Pins: torch's CPU float64 scaled-dot-product attention (library routine) with an explicit
bottom-right causal mask and explicitly repeated K/V heads for GQA; closed forms (one key, identical
values, identical keys); decode equals the last row of prefill."""
import numpy as np
import torch

import oracle
import workloads


def _sdpa(q, k, v, causal, scale=None):
    B, Lq, Hq, D = q.shape
    Lkv, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).repeat_interleave(g, dim=2).permute(0, 2, 1, 3).contiguous()
    vt = torch.from_numpy(v).repeat_interleave(g, dim=2).permute(0, 2, 1, 3).contiguous()
    mask = None
    if causal:
        i = torch.arange(Lq)[:, None]
        j = torch.arange(Lkv)[None, :]
        mask = j <= i + (Lkv - Lq)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def test_matches_torch_sdpa_float64():
    rng = np.random.default_rng(0)
    for (B, Lq, Lkv, Hq, Hkv, D, causal) in ((2, 9, 9, 4, 2, 16, True), (1, 3, 11, 6, 3, 8, True),
                                              (2, 5, 7, 2, 2, 32, False), (1, 1, 13, 8, 1, 128, True)):
        q = rng.standard_normal((B, Lq, Hq, D)) * 3
        k = rng.standard_normal((B, Lkv, Hkv, D))
        v = rng.standard_normal((B, Lkv, Hkv, D))
        o = oracle.attn_f64(q, k, v, causal)
        assert np.allclose(o, _sdpa(q, k, v, causal), rtol=1e-12, atol=1e-12)
        # explicit scale, and a row subset
        rows = np.array([[B - 1, Lq - 1, Hq - 1], [0, 0, 0]], np.int64)
        o2 = oracle.attn_f64(q, k, v, causal, scale=0.3, rows=rows)
        ref = _sdpa(q, k, v, causal, scale=0.3)
        assert np.allclose(o2[0], ref[B - 1, Lq - 1, Hq - 1], rtol=1e-12, atol=1e-12)
        assert np.allclose(o2[1], ref[0, 0, 0], rtol=1e-12, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 4, 2, 8))
    k = rng.standard_normal((1, 1, 2, 8))
    v = rng.standard_normal((1, 1, 2, 8))
    o = oracle.attn_f64(q, k, v, causal=False)
    assert np.array_equal(o, np.broadcast_to(v, o.shape))  # one key: O = v exactly (P = 1)
    k = rng.standard_normal((1, 6, 1, 8))
    v = np.broadcast_to(rng.standard_normal((1, 1, 1, 8)), (1, 6, 1, 8)).copy()
    o = oracle.attn_f64(rng.standard_normal((1, 6, 3, 8)), k, v, causal=True)
    assert np.allclose(o, v[0, 0, 0], rtol=1e-15, atol=1e-15)  # identical values
    k = np.broadcast_to(rng.standard_normal((1, 1, 1, 8)), (1, 6, 1, 8)).copy()
    v = rng.standard_normal((1, 6, 1, 8))
    o = oracle.attn_f64(rng.standard_normal((1, 6, 1, 8)), k, v, causal=True)
    for i in range(6):  # identical keys: uniform weights over the visible prefix
        assert np.allclose(o[0, i, 0], v[0, : i + 1, 0].mean(0), rtol=1e-14, atol=1e-14)


def test_decode_is_last_prefill_row_and_gqa():
    q16, qs = workloads.int16_cache_host(2, 12, 8, 128, seed=5)
    k16, ks = workloads.int16_cache_host(2, 12, 2, 128, seed=6)
    v16, vs = workloads.int16_cache_host(2, 12, 2, 128, seed=7)
    full = oracle.attn_i16_f64(q16, qs, k16, ks, v16, vs, causal=True)
    dec = oracle.attn_i16_f64(q16[:, -1:], qs[:, -1:], k16, ks, v16, vs, causal=True)
    assert np.array_equal(dec[:, 0], full[:, -1])
    # GQA equals MHA with each K/V head repeated for its group of 4 query heads
    k_rep = np.repeat(k16, 4, axis=2)
    v_rep = np.repeat(v16, 4, axis=2)
    mha = oracle.attn_i16_f64(q16, qs, k_rep, np.repeat(ks, 4, axis=2), v_rep, np.repeat(vs, 4, axis=2),
                              causal=True)
    assert np.array_equal(mha, full)


def test_dequant_exact():
    q = np.array([[[[32767, -32767, 1, 0]]]], np.int16)
    s = np.array([[[np.float32(1.0) / np.float32(3.0)]]], np.float32)
    x = oracle.dequant_i16(q, s)
    sd = float(np.float32(1.0) / np.float32(3.0))
    assert list(x[0, 0, 0]) == [32767 * sd, -32767 * sd, sd, 0.0]


def test_gather_pages_by_hand():
    # 2 sequences, page_size 4: sequence 0 = pages [2, 0], sequence 1 = page [1]
    pool = np.arange(3 * 4 * 2).reshape(3, 4, 2)  # [page, slot, feature]
    table = np.array([[2, 0], [1, -1]])
    g0 = oracle.gather_pages(pool, table[0], 6, 4)
    assert np.array_equal(g0, np.concatenate([pool[2], pool[0, :2]]))
    g1 = oracle.gather_pages(pool, table[1], 3, 4)
    assert np.array_equal(g1, pool[1, :3])
    # scatter then gather is the identity on a shuffled pool (the two are written independently)
    x = np.random.default_rng(0).integers(-9, 9, (3, 70, 2, 5)).astype(np.int16)
    lens = [70, 1, 33]
    P, tab = workloads.paged_layout(lens, 32, spare_pages=2, seed=1)
    pool = workloads.pages_from_contiguous(x, lens, tab, P, 32)
    for b, n in enumerate(lens):
        assert np.array_equal(oracle.gather_pages(pool, tab[b], n, 32), x[b, :n])


def test_paged_decode_matches_sdpa_on_the_contiguous_keys():
    B, Hq, Hkv, D, ps = 3, 8, 2, 128, 32
    lens = [1, 77, 130]
    Lmax = max(lens)
    q, qs = workloads.int16_cache_host(B, 1, Hq, D, seed=11)
    k, ks = workloads.int16_cache_host(B, Lmax, Hkv, D, seed=12)
    v, vs = workloads.int16_cache_host(B, Lmax, Hkv, D, seed=13)
    P, tab = workloads.paged_layout(lens, ps, seed=2)
    kp = workloads.pages_from_contiguous(k, lens, tab, P, ps)
    vp = workloads.pages_from_contiguous(v, lens, tab, P, ps)
    ksp = workloads.pages_from_contiguous(ks, lens, tab, P, ps, fill=1.0)
    vsp = workloads.pages_from_contiguous(vs, lens, tab, P, ps, fill=1.0)
    got = oracle.attn_paged_i16_f64(q[:, 0], qs[:, 0], kp, ksp, vp, vsp, tab, np.array(lens))
    for b, n in enumerate(lens):
        deq = lambda t, s: t[b:b + 1, :n].astype(np.float64) * s[b:b + 1, :n, :, None].astype(np.float64)
        want = _sdpa(q[b:b + 1].astype(np.float64) * qs[b:b + 1, :, :, None].astype(np.float64),
                     deq(k, ks), deq(v, vs), causal=False)
        assert np.allclose(got[b], want[0, 0], rtol=1e-12, atol=1e-12)
    # an empty sequence gives zeros
    z = oracle.attn_paged_i16_f64(q[:1, 0], qs[:1, 0], kp, ksp, vp, vsp, tab[:1], np.array([0]))
    assert np.all(z == 0)
