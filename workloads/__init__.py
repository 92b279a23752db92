"""Seeded synthetic inputs for the HEAL hot path.

This module is shared by the tests, the smoke check and the benchmark; it holds no step of the method
(no split, no quantisation, no product).  It only draws numbers with the shapes and value distributions of
the workloads:

* ``gemm_uniform``    -- FP32 A [M, K] and B^T [N, K], i.i.d. U[-1, 1] (the 256^3 correctness case).
* ``gemm_rowscaled``  -- FP32 N(0, 1) with every row of A and of B^T scaled by 10^U(-3, 3) (8192^3 case).
* ``llama_linear``    -- FP32 activations N(0, 1) [M, K] with a fixed 1 % of the K channels scaled x50,
                         and bf16 weights N(0, 0.02) [N, K] (Llama-3-8B projection shapes).
* ``qkv_fp32``        -- FP32 Q/K/V N(0, 1) * sigma_t, sigma_t ~ lognormal(0, 1) per (tensor, token).
* ``int16_cache``     -- an INT16 K/V cache of the same value distribution, drawn directly as integers
                         with per-(token, head) fp32 scales; what a decode step reads.

Seeds are plain integers; numpy's PCG64 (``default_rng``) draws every host array, so the oracle and the
GPU see identical bits.  The 2 GB decode cache is drawn on the device with torch's Philox generator and
slices are copied back for the oracle.
"""
from __future__ import annotations

import numpy as np

# Llama-3-8B projection shapes: (K, N) for M tokens.  q/o: 4096->4096, gate/up: 4096->14336, down:
# 14336->4096.
LLAMA3_8B_KN = ((4096, 4096), (4096, 14336), (14336, 4096))
LLAMA3_8B_M = (1, 16, 2048)


def gemm_uniform(M: int, N: int, K: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    A = rng.uniform(-1.0, 1.0, size=(M, K)).astype(np.float32)
    Bt = rng.uniform(-1.0, 1.0, size=(N, K)).astype(np.float32)
    return A, Bt


def gemm_rowscaled(M: int, N: int, K: int, seed: int = 4):
    """Rows of A (M of them) and of B (K of them, i.e. the k index of B^T) scaled by 10^U(-3, 3)."""
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K), dtype=np.float32)
    A *= (10.0 ** rng.uniform(-3.0, 3.0, size=(M, 1))).astype(np.float32)
    Bt = rng.standard_normal((N, K), dtype=np.float32)
    Bt *= (10.0 ** rng.uniform(-3.0, 3.0, size=(1, K))).astype(np.float32)
    return A, Bt


def outlier_channels(K: int, seed: int = 1, frac: float = 0.01) -> np.ndarray:
    """The fixed set of activation channels that carry outliers (1 % of K)."""
    rng = np.random.default_rng(seed + 1000)
    n = max(1, int(round(frac * K)))
    return np.sort(rng.choice(K, size=n, replace=False))


def llama_activations(M: int, K: int, seed: int = 1, outlier_gain: float = 50.0) -> np.ndarray:
    rng = np.random.default_rng(seed * 7919 + M * 31 + K)
    X = rng.standard_normal((M, K), dtype=np.float32)
    X[:, outlier_channels(K, seed)] *= np.float32(outlier_gain)
    return X


def llama_weights_bf16(N: int, K: int, seed: int = 1) -> np.ndarray:
    """bf16 weights N(0, 0.02) as uint16 bit patterns (torch's float32 -> bfloat16 cast, RNE)."""
    import torch

    rng = np.random.default_rng(seed * 104729 + N * 17 + K)
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    return torch.from_numpy(W).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def qkv_fp32(B: int, L: int, H: int, D: int, seed: int = 2):
    """Q, K, V fp32 [B, L, H, D]; each (tensor, batch, token) shares one lognormal(0, 1) scale."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        x = rng.standard_normal((B, L, H, D), dtype=np.float32)
        sig = np.exp(rng.standard_normal((B, L, 1, 1))).astype(np.float32)
        out.append(x * sig)
    return tuple(out)


INT16_SIGMA = 9362.0  # an N(0,1) row of 128 has max |x| near 3.5 sigma; 32767 / 3.5 = 9362


def int16_cache_host(B: int, L: int, H: int, D: int, seed: int = 3):
    """A synthetic INT16 tensor [B, L, H, D] with per-(b, token, head) fp32 scales [B, L, H].

    Integers ~ round(N(0, 9362)) clipped to +-32767 (the spread of a symmetric per-row INT16 code of a
    Gaussian row); scales sigma_t / 9362 with sigma_t ~ lognormal(0, 1) per (b, token), so s * q has the
    distribution N(0, 1) * sigma_t of the other attention inputs."""
    rng = np.random.default_rng(seed)
    q = np.clip(np.rint(rng.standard_normal((B, L, H, D)) * INT16_SIGMA), -32767, 32767).astype(np.int16)
    sig = np.exp(rng.standard_normal((B, L, 1)))
    s = np.broadcast_to(sig / INT16_SIGMA, (B, L, H)).astype(np.float32)
    return q, np.ascontiguousarray(s)


def int16_cache_device(B: int, L: int, H: int, D: int, seed: int = 3, device: str = "cuda"):
    """The same distribution as ``int16_cache_host``, drawn on the device (torch Philox) for the 2 GB
    decode cache.  Returns torch tensors (q int16 [B, L, H, D], s fp32 [B, L, H])."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = torch.empty((B, L, H, D), dtype=torch.int16, device=device)
    chunk = max(1, (1 << 27) // (L * H * D))
    for b0 in range(0, B, chunk):
        b1 = min(B, b0 + chunk)
        t = torch.randn((b1 - b0, L, H, D), generator=g, device=device, dtype=torch.float32)
        q[b0:b1] = torch.round(t * INT16_SIGMA).clamp_(-32767, 32767).to(torch.int16)
        del t
    sig = torch.exp(torch.randn((B, L, 1), generator=g, device=device, dtype=torch.float32))
    s = (sig / INT16_SIGMA).expand(B, L, H).contiguous()
    return q, s


def paged_layout(seq_lens, page_size: int, spare_pages: int = 3, seed: int = 7):
    """A shuffled page assignment for sequences of the given lengths: returns (num_pages, block_table
    [B, max_pages] int32).  Every page of every sequence is a distinct pool page in random order, the pool
    holds spare_pages unused pages besides, and table columns past a sequence's pages hold -1."""
    rng = np.random.default_rng(seed)
    seq_lens = [int(n) for n in seq_lens]
    need = [(n + page_size - 1) // page_size for n in seq_lens]
    max_pages = max(1, max(need) if need else 1)
    num_pages = sum(need) + spare_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((len(seq_lens), max_pages), -1, np.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[at:at + n]
        at += n
    return num_pages, table


def pages_from_contiguous(x: np.ndarray, seq_lens, table: np.ndarray, num_pages: int, page_size: int,
                          fill=0):
    """Scatter a contiguous per-sequence tensor x [B, L, ...] into a page pool [num_pages, page_size, ...]
    following `table` (key j of sequence b -> slot j % page_size of page table[b, j // page_size]); slots
    no sequence uses hold `fill`."""
    pool = np.full((num_pages, page_size) + x.shape[2:], fill, x.dtype)
    for b, n in enumerate(seq_lens):
        for j0 in range(0, int(n), page_size):
            j1 = min(int(n), j0 + page_size)
            pool[table[b, j0 // page_size], :j1 - j0] = x[b, j0:j1]
    return pool


def massive_channels(M: int, K: int, frac: float = 0.01, big: float = 1e5, small: float = 1e-5, seed: int = 9):
    """Activations with massive channels: small * N(0, 1) everywhere, except a fixed frac of the K channels
    that carry +-big * U(0.5, 1) in every row.  Returns (x fp32 [M, K], the outlier channel indices)."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((M, K)) * small).astype(np.float32)
    idx = np.sort(rng.choice(K, size=max(1, int(round(frac * K))), replace=False))
    x[:, idx] = (rng.choice([-1.0, 1.0], size=(M, idx.size)) * rng.uniform(0.5, 1.0, (M, idx.size)) * big
                 ).astype(np.float32)
    return x, idx
