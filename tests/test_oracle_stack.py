"""Pins of the FP64 decoder-stack oracle (``oracle.stack``) on the CPU: rotary-embedding invariants (identity
at position 0, norm preservation, dot products that depend only on the position difference), RMSNorm's unit
mean square, the causal first query seeing one key, the KV-cached incremental forward equal to one full
forward, and a tiny model against an independent torch float64 forward (its scaled_dot_product_attention with
a causal mask, repeated key/value heads, F.silu)."""
import numpy as np
import torch

from oracle import stack


def _weights(rng, layers, d, hq, hkv, f, vocab):
    def bf16(shape):
        x = torch.from_numpy(rng.standard_normal(shape) * 0.02).to(torch.bfloat16)
        return x.view(torch.int16).numpy().view(np.uint16)
    w = {"emb": bf16((vocab, d)), "head": bf16((vocab, d))}
    for l in range(layers):
        w[f"{l}.wq"], w[f"{l}.wk"], w[f"{l}.wv"] = bf16((hq * 128, d)), bf16((hkv * 128, d)), bf16((hkv * 128, d))
        w[f"{l}.wo"] = bf16((d, hq * 128))
        w[f"{l}.wg"], w[f"{l}.wu"], w[f"{l}.wd"] = bf16((f, d)), bf16((f, d)), bf16((d, f))
    return w


def test_bf16_values_exact():
    x = torch.randn(1000, dtype=torch.float32).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(stack.bf16_to_f64(bits), x.to(torch.float64).numpy())


def test_rope_invariants():
    rng = np.random.default_rng(0)
    cos, sin = stack.rope_tables(64, 5e5)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    assert np.allclose(stack.rope(q, cos[:1], sin[:1]), q, rtol=0, atol=0)  # position 0: identity
    r = stack.rope(q, cos[37:38], sin[37:38])
    assert np.isclose(np.linalg.norm(r), np.linalg.norm(q), rtol=1e-14)
    dot = lambda m, n: float(np.sum(stack.rope(q, cos[m:m + 1], sin[m:m + 1]) * stack.rope(k, cos[n:n + 1], sin[n:n + 1])))
    assert np.isclose(dot(20, 5), dot(35, 20), rtol=1e-12) and np.isclose(dot(20, 5), dot(15, 0), rtol=1e-12)
    assert not np.isclose(dot(20, 5), dot(20, 6), rtol=1e-6)  # and it does depend on the difference


def test_rms_norm_unit_mean_square():
    x = np.random.default_rng(1).standard_normal((5, 4096)) * 7
    y = stack.rms_norm(x, 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)


def test_incremental_equals_full_and_first_query():
    rng = np.random.default_rng(2)
    w = _weights(rng, 2, 256, 4, 2, 512, 300)
    ids = rng.integers(0, 300, 9)
    full = stack.Stack(w, 2, 4, 2)
    h_full, lg_full = full.forward(ids, 0)
    inc = stack.Stack(w, 2, 4, 2)
    inc.forward(ids[:5], 0)
    for t in range(5, 9):
        h_inc, lg_inc = inc.forward(ids[t:t + 1], t)
    assert np.allclose(h_inc, h_full, rtol=0, atol=1e-12) and np.allclose(lg_inc, lg_full, rtol=0, atol=1e-12)
    # the first query of a causal prefill sees only key 0: its attention output is that key's value
    one = stack.Stack(w, 1, 4, 2)
    q = rng.standard_normal((3, 4, 128))
    one.k[0] = rng.standard_normal((3, 2, 128))
    one.v[0] = rng.standard_normal((3, 2, 128))
    out = one.attention(q, 0, 0)
    assert np.allclose(out[0, 0], one.v[0][0, 0], rtol=0, atol=1e-15)
    assert np.allclose(out[0, 3], one.v[0][0, 1], rtol=0, atol=1e-15)  # query head 3 reads kv head 1


def test_tiny_model_against_torch_float64():
    import torch.nn.functional as F
    rng = np.random.default_rng(3)
    L, d, hq, hkv, f, vocab, T = 2, 256, 4, 2, 384, 257, 11
    w = _weights(rng, L, d, hq, hkv, f, vocab)
    ids = rng.integers(0, vocab, T)
    h_ref, lg_ref = stack.Stack(w, L, hq, hkv).forward(ids, 0)
    W = {k: torch.from_numpy(stack.bf16_to_f64(v)) for k, v in w.items()}
    inv = 5e5 ** (-torch.arange(64, dtype=torch.float64) / 64)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None, :]
    cos, sin = torch.cat([ang.cos(), ang.cos()], 1), torch.cat([ang.sin(), ang.sin()], 1)
    def rot(x):  # x [H, T, 128]: x * cos + rotate_half(x) * sin
        return x * cos + torch.cat([-x[..., 64:], x[..., :64]], -1) * sin
    def norm(x):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + 1e-5)
    x = W["emb"][torch.from_numpy(ids)]
    for l in range(L):
        h = norm(x)
        q = (h @ W[f"{l}.wq"].T).view(T, hq, 128).transpose(0, 1)
        k = (h @ W[f"{l}.wk"].T).view(T, hkv, 128).transpose(0, 1).repeat_interleave(hq // hkv, 0)
        v = (h @ W[f"{l}.wv"].T).view(T, hkv, 128).transpose(0, 1).repeat_interleave(hq // hkv, 0)
        a = F.scaled_dot_product_attention(rot(q)[None], rot(k)[None], v[None], is_causal=True)[0]
        x = x + a.transpose(0, 1).reshape(T, hq * 128) @ W[f"{l}.wo"].T
        h = norm(x)
        x = x + (F.silu(h @ W[f"{l}.wg"].T) * (h @ W[f"{l}.wu"].T)) @ W[f"{l}.wd"].T
    hn = norm(x[-1])
    lg = W["head"] @ hn
    assert np.allclose(h_ref, hn.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(lg_ref, lg.numpy(), rtol=0, atol=1e-12)
