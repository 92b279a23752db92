"""FP64 forward of a Llama-style decoder stack: the reference for the model-level check of the HEAL path
(a random-initialised stack whose greedy argmax the 16-bit paths should reproduce).  TEST INFRASTRUCTURE
ONLY, like the rest of ``oracle``.

The block is the one the check names: token embedding; per layer RMSNorm -> Q, K, V projections -> rotary
embedding on Q and K -> causal grouped-query attention -> output projection -> residual; RMSNorm -> SwiGLU
feed-forward (gate, up, down) -> residual; a final RMSNorm and the LM head.  Conventions where the
description leaves them open (each listed with its reason in the design notes): RMSNorm with unit weight and
eps 1e-5; rotary pairs (i, i + 64) of each 128-wide head with angle pos * theta^(-i / 64), theta = 5e5;
query head h reads key/value head h // (Hq / Hkv); softmax scale 1 / sqrt(128).  Every value is FP64; the
weights are bf16 and enter exactly.  Nothing here is quantised: this is the model the 16-bit paths
approximate.
"""
from __future__ import annotations

import numpy as np

D_HEAD = 128


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (uint16)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rms_norm(x: np.ndarray, eps: float) -> np.ndarray:
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope_tables(positions: int, theta: float) -> tuple[np.ndarray, np.ndarray]:
    """cos and sin [positions, 64] of the angles pos * theta^(-i / 64) in FP64."""
    inv = theta ** (-np.arange(64, dtype=np.float64) / 64.0)
    ang = np.arange(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """x [T, H, 128]; cos / sin [T, 64] for the tokens' positions."""
    a, b = x[..., :64], x[..., 64:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


class Stack:
    """The FP64 model.  ``w`` maps names to bf16 bit arrays: "emb" [V, d], "head" [V, d], and per layer l
    "l.wq" [Hq*128, d], "l.wk" / "l.wv" [Hkv*128, d], "l.wo" [d, Hq*128], "l.wg" / "l.wu" [F, d], "l.wd" [d, F]
    (every matrix maps its input along the last axis: y = x @ W.T)."""

    def __init__(self, w: dict, layers: int, hq: int, hkv: int, eps: float = 1e-5, theta: float = 5e5,
                 max_len: int = 1024):
        self.w = dict(w)  # its own table: widened matrices leave it (the caller's table is untouched)
        self.layers, self.hq, self.hkv, self.eps = layers, hq, hkv, eps
        self.cos, self.sin = rope_tables(max_len, theta)
        self._f64 = {}
        self.k = [np.zeros((0, hkv, D_HEAD)) for _ in range(layers)]
        self.v = [np.zeros((0, hkv, D_HEAD)) for _ in range(layers)]

    def W(self, name: str) -> np.ndarray:
        """FP64 copy of matrix ``name``, made on first use; the bf16 source is then dropped from ``w`` (every
        decode step needs every matrix again, so widening on each use would convert all weights per token)."""
        if name not in self._f64:
            self._f64[name] = bf16_to_f64(self.w.pop(name))
        return self._f64[name]

    def attention(self, q: np.ndarray, l: int, pos0: int) -> np.ndarray:
        """q [T, Hq, 128] at positions pos0..pos0+T-1 over the cache of layer l (keys 0..pos0+T-1)."""
        T = q.shape[0]
        K, V = self.k[l], self.v[l]
        g = self.hq // self.hkv
        out = np.empty_like(q)
        for h in range(self.hq):
            s = q[:, h, :] @ K[:, h // g, :].T / np.sqrt(D_HEAD)  # [T, L]
            mask = np.arange(K.shape[0])[None, :] > (pos0 + np.arange(T))[:, None]
            s[mask] = -np.inf
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[:, h, :] = (p @ V[:, h // g, :]) / p.sum(axis=1, keepdims=True)
        return out

    def forward(self, ids: np.ndarray, pos0: int):
        """Run tokens ``ids`` at positions pos0.. (appending to the cache); returns (final normalised hidden of
        the last token [d], its logits [V])."""
        T = len(ids)
        x = bf16_to_f64(self.w["emb"][np.asarray(ids)])  # only the rows looked up
        cos, sin = self.cos[pos0:pos0 + T], self.sin[pos0:pos0 + T]
        for l in range(self.layers):
            h = rms_norm(x, self.eps)
            q = (h @ self.W(f"{l}.wq").T).reshape(T, self.hq, D_HEAD)
            k = (h @ self.W(f"{l}.wk").T).reshape(T, self.hkv, D_HEAD)
            v = (h @ self.W(f"{l}.wv").T).reshape(T, self.hkv, D_HEAD)
            q, k = rope(q, cos, sin), rope(k, cos, sin)
            self.k[l] = np.concatenate([self.k[l], k])
            self.v[l] = np.concatenate([self.v[l], v])
            a = self.attention(q, l, pos0).reshape(T, self.hq * D_HEAD)
            x = x + a @ self.W(f"{l}.wo").T
            h = rms_norm(x, self.eps)
            gte, up = h @ self.W(f"{l}.wg").T, h @ self.W(f"{l}.wu").T
            x = x + (gte / (1.0 + np.exp(-gte)) * up) @ self.W(f"{l}.wd").T
        hn = rms_norm(x[-1], self.eps)
        return hn, self.W("head") @ hn
