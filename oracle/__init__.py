"""The plain CPU oracle of the HEAL hot path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` import this
package.  The product path (``error_compensated_gemm_amd``) never does, and it shares no code with it:
the oracle is plain C (``heal_oracle.c``, built with gcc, no HIP headers) behind the numpy wrappers below.

Sources, cited by page title and section:
  [TS]  gist.science explainer "Demystifying Numerical Instability in LLM Inference: Achieving
        Reproducible Inference for Mission-Critical Tasks with HEAL", "Technical Summary";
        [TS 2A] INT16 quantisation / Dual-FP16 unpack, [TS 2B] algebraic error compensation.
  [ABS] the authors' abstract, arXiv 2606.21023 v2.

Every function says which passage it follows; the readings adopted where the pages are silent are
spelled out in ``heal_oracle.c``.  Parity status: every function is pinned by the ``-m "not gpu"``
tests in ``tests/test_oracle_*.py`` (library special cases, closed forms, exhaustive enumeration,
brute force on tiny inputs); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "heal_oracle.c")
_LIB = os.path.join(_HERE, "libheal_oracle.so")

F16 = 2
BF16 = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: IEEE arithmetic, no contraction, no fast-math."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-frounding-math", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        L.orc_f16_bits.restype = ctypes.c_uint16
        L.orc_f16_bits.argtypes = [ctypes.c_float]
        L.orc_bf16_bits.restype = ctypes.c_uint16
        L.orc_bf16_bits.argtypes = [ctypes.c_float]
        L.orc_f16_value.restype = ctypes.c_double
        L.orc_f16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_f16_bits_array.argtypes = [p, i64, p]
        L.orc_bf16_bits_array.argtypes = [p, i64, p]
        L.orc_split_f32.argtypes = [p, i64, i64, i64, ctypes.c_int, ctypes.c_int, p, p, i64, p]
        L.orc_split_bf16.argtypes = [p, i64, i64, i64, ctypes.c_int, ctypes.c_int, p, p, i64, p]
        L.orc_split_i16.argtypes = [p, i64, i64, i64, p, p, i64]
        L.orc_unpack_i16.argtypes = [p, i64, i64, i64, ctypes.c_int, p, p, i64]
        L.orc_quant_i16.argtypes = [p, i64, i64, i64, i64, p, p]
        L.orc_gemm_f64.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64]
        L.orc_gemm_f64_points.argtypes = [i64, p, i64, p, i64, i64, p, p, p]
        L.orc_gemm_emul.argtypes = [i64, i64, i64, p, p, p, i64, p, p, p, i64, ctypes.c_int, p, p, i64]
        L.orc_attn_f64.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, ctypes.c_int, ctypes.c_double,
                                   i64, p, p, p, p]
        L.orc_dequant_i16.argtypes = [i64, i64, i64, i64, p, p, p, p, p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------------------------- conversions
def f16_bits(x: np.ndarray) -> np.ndarray:
    """IEEE binary16 round-to-nearest-even of fp32 values, returned as uint16 bit patterns."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f16_bits_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 round-to-nearest-even of fp32 values, returned as uint16 bit patterns."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_bits_array(_ptr(x), x.size, _ptr(out))
    return out


def f16_value(b: int) -> float:
    return lib().orc_f16_value(int(b))


def bf16_value(b: int) -> float:
    return lib().orc_bf16_value(int(b))


def part_values(bits: np.ndarray, part: int) -> np.ndarray:
    """Exact float64 values of a uint16 array of FP16 (part=F16) or bf16 (part=BF16) patterns."""
    bits = np.asarray(bits, np.uint16)
    uniq, inv = np.unique(bits, return_inverse=True)
    f = lib().orc_f16_value if part == F16 else lib().orc_bf16_value
    vals = np.array([f(int(u)) for u in uniq], np.float64)
    return vals[inv].reshape(bits.shape)


# ----------------------------------------------------------------------------------------------------- split
def split_f32(x: np.ndarray, part: int = F16, prescale: bool = True, residual: bool = True):
    """[TS 2B Mechanism] primary 16-bit value + residual, with the power-of-two row prescale standing for
    [TS 2B Overflow Handling].  Returns (hi_bits, lo_bits or None, exps int32 [rows])."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    hi = np.empty((rows, cols), np.uint16)
    lo = np.empty((rows, cols), np.uint16) if residual else None
    e = np.empty(rows, np.int32)
    lib().orc_split_f32(_ptr(x), rows, cols, cols, part, int(prescale), _ptr(hi), _ptr(lo), cols, _ptr(e))
    return hi, lo, e


def split_bf16(x_bits: np.ndarray, part: int = F16, prescale: bool = True, residual: bool = False):
    """The same split applied to bf16 weights (uint16 patterns in)."""
    x_bits = _c(x_bits, np.uint16)
    rows, cols = x_bits.shape
    hi = np.empty((rows, cols), np.uint16)
    lo = np.empty((rows, cols), np.uint16) if residual else None
    e = np.empty(rows, np.int32)
    lib().orc_split_bf16(_ptr(x_bits), rows, cols, cols, part, int(prescale), _ptr(hi), _ptr(lo), cols,
                         _ptr(e))
    return hi, lo, e


def split_i16(q: np.ndarray):
    """[TS 2A Mechanism] Dual-FP16 unpack (byte split): FP16 bits of hi = q >> 8 and lo = q & 0xFF."""
    q = _c(q, np.int16)
    rows, cols = q.shape
    hi = np.empty((rows, cols), np.uint16)
    lo = np.empty((rows, cols), np.uint16)
    lib().orc_split_i16(_ptr(q), rows, cols, cols, _ptr(hi), _ptr(lo), cols)
    return hi, lo


DUAL_READINGS = {"byte": 0, "shift10": 1, "float": 2}


def unpack_i16(q: np.ndarray, reading: str):
    """[TS 2A Mechanism] Dual-FP16 unpack under one of three readings of the pair (FP16 bits out):
    "byte" hi = floor(q / 256), lo = q mod 256; "shift10" hi = floor(q / 1024), lo = q mod 1024;
    "float" hi = fp16_rn(q), lo = 1024 (q - hi)."""
    q = _c(q, np.int16)
    rows, cols = q.shape
    hi = np.empty((rows, cols), np.uint16)
    lo = np.empty((rows, cols), np.uint16)
    lib().orc_unpack_i16(_ptr(q), rows, cols, cols, DUAL_READINGS[reading], _ptr(hi), _ptr(lo), cols)
    return hi, lo


# -------------------------------------------------------------------------------------------------- quantise
def quant_i16(x: np.ndarray):
    """[TS 2A Solution] INT16 quantisation per (token, head).  x: [T, H, D] fp32 -> (q int16, s fp32)."""
    x = _c(x, np.float32)
    T, H, D = x.shape
    q = np.empty((T, H, D), np.int16)
    s = np.empty((T, H), np.float32)
    lib().orc_quant_i16(_ptr(x), T, H, D, H * D, _ptr(q), _ptr(s))
    return q, s


# ------------------------------------------------------------------------------------------------------ GEMM
def gemm_f64(A: np.ndarray, Bt: np.ndarray) -> np.ndarray:
    """Definition of the compensated GEMM's target: C = A @ Bt.T in FP64 (plain triple loop)."""
    A = _c(A, np.float64)
    Bt = _c(Bt, np.float64)
    M, K = A.shape
    N = Bt.shape[0]
    C = np.empty((M, N), np.float64)
    lib().orc_gemm_f64(M, N, K, _ptr(A), K, _ptr(Bt), K, _ptr(C), N)
    return C


def gemm_f64_points(A: np.ndarray, Bt: np.ndarray, ii: np.ndarray, jj: np.ndarray) -> np.ndarray:
    """C[ii[p], jj[p]] of the FP64 definition, one dot product per requested position."""
    A = _c(A, np.float64)
    Bt = _c(Bt, np.float64)
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    out = np.empty(ii.shape, np.float64)
    lib().orc_gemm_f64_points(A.shape[1], _ptr(A), A.shape[1], _ptr(Bt), Bt.shape[1], ii.size, _ptr(ii),
                              _ptr(jj), _ptr(out))
    return out


def gemm_emul(ah, al, ea, bh, bl, eb, part: int = F16):
    """Emulation level: exact FP64 sum of the method's 16-bit products, and the magnitude sum G.
    Returns (C_e, G), both [M, N] float64."""
    ah = _c(ah, np.uint16)
    bh = _c(bh, np.uint16)
    al = None if al is None else _c(al, np.uint16)
    bl = None if bl is None else _c(bl, np.uint16)
    ea = None if ea is None else _c(ea, np.int32)
    eb = None if eb is None else _c(eb, np.int32)
    M, K = ah.shape
    N = bh.shape[0]
    C = np.empty((M, N), np.float64)
    G = np.empty((M, N), np.float64)
    lib().orc_gemm_emul(M, N, K, _ptr(ah), _ptr(al), _ptr(ea), K, _ptr(bh), _ptr(bl), _ptr(eb), K, part,
                        _ptr(C), _ptr(G), N)
    return C, G


# ------------------------------------------------------------------------------------------------- attention
def dequant_i16(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """x = s * q in float64 for q [B, L, H, D] int16 and s [B, L, H] fp32 (exact)."""
    q = _c(q, np.int16)
    s = _c(s, np.float32)
    B, L, H, D = q.shape
    out = np.empty((B, L, H, D), np.float64)
    qs = np.array([L * H * D, H * D, D], np.int64)
    ss = np.array([L * H, H, 1], np.int64)
    lib().orc_dequant_i16(B, L, H, D, _ptr(q), _ptr(qs), _ptr(s), _ptr(ss), _ptr(out))
    return out


def attn_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float | None = None,
             rows=None) -> np.ndarray:
    """FP64 attention on real-valued q [B, Lq, Hq, D], k/v [B, Lkv, Hkv, D].

    rows: None for every (b, i, h), else an int64 array [R, 3] of (b, i, h).  Returns O with shape
    [B, Lq, Hq, D] (rows=None) or [R, D]."""
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    v = _c(v, np.float64)
    B, Lq, Hq, D = q.shape
    Lkv, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(np.float64(D))
    full = rows is None
    if full:
        bb, ii, hh = np.meshgrid(np.arange(B), np.arange(Lq), np.arange(Hq), indexing="ij")
        rows = np.stack([bb.ravel(), ii.ravel(), hh.ravel()], 1)
    rows = _c(rows, np.int64)
    rb, ri, rh = (_c(rows[:, c], np.int64) for c in range(3))
    out = np.empty((rows.shape[0], D), np.float64)
    qs = np.array([Lq * Hq * D, Hq * D, D], np.int64)
    ks = np.array([Lkv * Hkv * D, Hkv * D, D], np.int64)
    lib().orc_attn_f64(Lq, Lkv, Hq, Hkv, D, _ptr(q), _ptr(qs), _ptr(k), _ptr(v), _ptr(ks), int(causal),
                       float(scale), rows.shape[0], _ptr(rb), _ptr(ri), _ptr(rh), _ptr(out))
    return out.reshape(B, Lq, Hq, D) if full else out


def attn_i16_f64(q, qs, k, ks, v, vs, causal: bool, scale: float | None = None, rows=None):
    """[TS 2A] attention graded on the dequantised INT16 inputs x = s * q (reading R-attn)."""
    return attn_f64(dequant_i16(q, qs), dequant_i16(k, ks), dequant_i16(v, vs), causal, scale, rows)


def gather_pages(pool: np.ndarray, table_row: np.ndarray, seq_len: int, page_size: int) -> np.ndarray:
    """The first seq_len keys of one sequence from a page pool [P, page_size, ...]: key j is slot
    j % page_size of page table_row[j // page_size] (the paged layout of the decode KV cache)."""
    j = np.arange(int(seq_len))
    return pool[np.asarray(table_row)[j // page_size], j % page_size]


def attn_paged_i16_f64(q, qs, k_pages, ks_pages, v_pages, vs_pages, block_table, seq_lens, scale=None):
    """Decode attention (one query token per sequence) over a paged INT16 cache, graded like
    attn_i16_f64: each sequence's keys are gathered from its pages and the FP64 definition is applied to
    the dequantised values.  q [B, Hq, D] int16, qs [B, Hq]; returns [B, Hq, D] (0 for an empty sequence)."""
    B, Hq, D = q.shape
    ps = k_pages.shape[1]
    out = np.zeros((B, Hq, D), np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        k = gather_pages(k_pages, block_table[b], n, ps)[None]
        ks = gather_pages(ks_pages, block_table[b], n, ps)[None]
        v = gather_pages(v_pages, block_table[b], n, ps)[None]
        vs = gather_pages(vs_pages, block_table[b], n, ps)[None]
        out[b] = attn_i16_f64(q[b][None, None], qs[b][None, None], k, ks, v, vs, causal=False, scale=scale)[0, 0]
    return out


def channel_exponents(x: np.ndarray, threshold_log2: int) -> np.ndarray:
    """[TS 2B Overflow Handling] read as exact power-of-two scales of the few outlier columns only (the pages
    give no rule; this one is the plainest): m_c = max_r |x[r, c]|; columns with ilogb(m_c) > T get
    T - ilogb(m_c), the others 0."""
    x = np.asarray(x, np.float64)
    m = np.max(np.abs(x), axis=0) if x.shape[0] else np.zeros(x.shape[1])
    _, e = np.frexp(m)  # m = f 2^e with f in [0.5, 1): ilogb(m) = e - 1
    il = e - 1
    return np.where((m > 0) & (il > threshold_log2), threshold_log2 - il, 0).astype(np.int32)


def scale_columns(x_values: np.ndarray, col_exps: np.ndarray, sign: int) -> np.ndarray:
    """x'[r, c] = fl32(x[r, c] 2^(sign col_exps[c])): the product is exact in FP64 and rounded once to FP32
    (round-to-nearest-even, gradual underflow)."""
    x = np.asarray(x_values, np.float64)
    return (x * np.ldexp(1.0, sign * np.asarray(col_exps, np.int64))[None, :]).astype(np.float32)
