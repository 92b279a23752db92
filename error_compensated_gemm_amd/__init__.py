"""Python binding of libheal, the HEAL hot path on AMD Instinct MI355X (gfx950).

The four calls of ``include/heal.h`` under the same names.  This module only marshals arguments: it
allocates outputs with torch (device memory), passes raw device pointers and the current HIP stream,
and raises ``RuntimeError`` with the library's status text on any error.  Every step of the path runs in
the HIP kernels of ``libheal.so``; there is no CPU or PyTorch fallback, and ``load()`` fails loudly when
the library has not been built.

Sources: gist.science explainer "Demystifying Numerical Instability in LLM Inference: Achieving
Reproducible Inference for Mission-Critical Tasks with HEAL", Technical Summary, sections 2.A (INT16
quantisation, Dual-FP16 unpack) and 2.B (algebraic error compensation, overflow handling).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libheal.so")

HEAL_F32, HEAL_BF16, HEAL_F16, HEAL_I16 = 0, 1, 2, 3
_PARTS = {"f16": HEAL_F16, "bf16": HEAL_BF16}
HEAL_DUAL_BYTE, HEAL_DUAL_SHIFT10, HEAL_DUAL_FLOAT = 0, 1, 2
_DUAL = {"byte": HEAL_DUAL_BYTE, "shift10": HEAL_DUAL_SHIFT10, "float": HEAL_DUAL_FLOAT}

_lib = None


class HealAttnArgs(ctypes.Structure):
    """Mirror of heal_attn_args in include/heal.h."""

    _fields_ = [
        ("batch", ctypes.c_int64), ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64),
        ("n_q_heads", ctypes.c_int64), ("n_kv_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("q_scale", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("q_strides", ctypes.c_int64 * 3), ("kv_strides", ctypes.c_int64 * 3),
        ("qs_strides", ctypes.c_int64 * 3), ("kvs_strides", ctypes.c_int64 * 3),
        ("o_strides", ctypes.c_int64 * 3),
        ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("dual_split", ctypes.c_int32),
        ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class HealPagedDecodeArgs(ctypes.Structure):
    """Mirror of heal_paged_decode_args in include/heal.h."""

    _fields_ = [
        ("batch", ctypes.c_int64), ("n_q_heads", ctypes.c_int64), ("n_kv_heads", ctypes.c_int64),
        ("head_dim", ctypes.c_int64), ("page_size", ctypes.c_int64), ("num_pages", ctypes.c_int64),
        ("max_pages_per_seq", ctypes.c_int64), ("max_kv_len", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("q_scale", ctypes.c_void_p), ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("q_strides", ctypes.c_int64 * 2), ("qs_strides", ctypes.c_int64 * 2),
        ("kv_strides", ctypes.c_int64 * 3), ("kvs_strides", ctypes.c_int64 * 3),
        ("o_strides", ctypes.c_int64 * 2), ("bt_stride", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float), ("dual_split", ctypes.c_int32),
        ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


def load():
    """Load libheal.so (built in-tree by ``build.build()``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libheal.so not built ({LIB_PATH}); run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.heal_status_str.restype = ctypes.c_char_p
    L.heal_status_str.argtypes = [i32]
    L.heal_abi_version.restype = i32
    L.heal_abi_version.argtypes = []
    L.heal_split.restype = i32
    L.heal_split.argtypes = [p, i32, i64, i64, i64, i32, p, p, i64, p, p]
    L.heal_row_exponents.restype = i32
    L.heal_row_exponents.argtypes = [p, i64, i64, i64, p, p]
    L.heal_gemm_comp_f32a.restype = i32
    L.heal_gemm_comp_f32a.argtypes = [i64, i64, i64, p, i64, p, p, p, p, i64, p, i64, p]
    L.heal_unpack_i16.restype = i32
    L.heal_unpack_i16.argtypes = [p, i64, i64, i64, i32, p, p, i64, p]
    L.heal_gemm_comp.restype = i32
    L.heal_gemm_comp.argtypes = [i64, i64, i64, p, p, p, i64, p, p, p, i64, i32, p, i64, p]
    L.heal_channel_exponents.restype = i32
    L.heal_channel_exponents.argtypes = [p, i64, i64, i64, i32, p, p]
    L.heal_split_scaled.restype = i32
    L.heal_split_scaled.argtypes = [p, i32, i64, i64, i64, i32, p, p, i64, p, p, i32, p]
    L.heal_gemm_comp_quant_i16.restype = i32
    L.heal_gemm_comp_quant_i16.argtypes = [i64, i64, i64, p, p, p, i64, p, p, p, i64, i32, p, i64, p, i64, p]
    L.heal_gemm_comp_variant.restype = ctypes.c_char_p
    L.heal_gemm_comp_variant.argtypes = [i64, i64, i64, i32]
    L.heal_gemm_comp_splitk.restype = i32
    L.heal_gemm_comp_splitk.argtypes = [i64, i64, i64, p, p, p, i64, p, p, p, i64, i32, p, i64, p, ctypes.c_size_t, p]
    L.heal_gemm_comp_workspace_bytes.restype = ctypes.c_size_t
    L.heal_gemm_comp_workspace_bytes.argtypes = [i64, i64, i64, i32]
    L.heal_gemm_comp_splitk_slices.restype = i32
    L.heal_gemm_comp_splitk_slices.argtypes = [i64, i64, i64, i32]
    L.heal_gemm_comp_f32a_splitk.restype = i32
    L.heal_gemm_comp_f32a_splitk.argtypes = [i64, i64, i64, p, i64, p, p, p, p, i64, p, i64, p, ctypes.c_size_t, p]
    L.heal_gemm_comp_f32a_workspace_bytes.restype = ctypes.c_size_t
    L.heal_gemm_comp_f32a_workspace_bytes.argtypes = [i64, i64, i64, i32]
    L.heal_gemm_comp_f32a_splitk_slices.restype = i32
    L.heal_gemm_comp_f32a_splitk_slices.argtypes = [i64, i64, i64, i32]
    L.heal_qkv_quant_i16.restype = i32
    L.heal_qkv_quant_i16.argtypes = [p, i64, i64, i64, i64, p, i64, p, i64, p]
    L.heal_attn_workspace_bytes.restype = ctypes.c_size_t
    L.heal_attn_workspace_bytes.argtypes = [ctypes.POINTER(HealAttnArgs)]
    L.heal_attn_dual_fp16.restype = i32
    L.heal_attn_dual_fp16.argtypes = [ctypes.POINTER(HealAttnArgs), p]
    L.heal_attn_dual_fp16_noalloc.restype = i32
    L.heal_attn_dual_fp16_noalloc.argtypes = [ctypes.POINTER(HealAttnArgs), p]
    L.heal_attn_paged_workspace_bytes.restype = ctypes.c_size_t
    L.heal_attn_paged_workspace_bytes.argtypes = [ctypes.POINTER(HealPagedDecodeArgs)]
    L.heal_attn_decode_paged.restype = i32
    L.heal_attn_decode_paged.argtypes = [ctypes.POINTER(HealPagedDecodeArgs), p]
    _lib = L
    return L


EXPORTED = ("heal_status_str", "heal_abi_version", "heal_split", "heal_gemm_comp", "heal_gemm_comp_variant",
            "heal_qkv_quant_i16", "heal_attn_workspace_bytes", "heal_attn_dual_fp16",
            "heal_attn_paged_workspace_bytes", "heal_attn_decode_paged", "heal_gemm_comp_quant_i16",
            "heal_channel_exponents", "heal_split_scaled", "heal_unpack_i16", "heal_row_exponents",
            "heal_gemm_comp_f32a", "heal_gemm_comp_splitk", "heal_gemm_comp_workspace_bytes",
            "heal_gemm_comp_splitk_slices", "heal_attn_dual_fp16_noalloc", "heal_gemm_comp_f32a_splitk",
            "heal_gemm_comp_f32a_workspace_bytes", "heal_gemm_comp_f32a_splitk_slices")
HEAL_ATTN_NOALLOC_MAX_WORKSPACE = 8 << 20


def _check(status: int):
    if status != 0:
        raise RuntimeError(load().heal_status_str(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ld(t) -> int:
    """leading dimension (elements) of a row-major 2-D view"""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


# -------------------------------------------------------------------------------------------------- heal_split
def heal_split(x, part: str = "f16", prescale: bool = True, residual: bool = True, hi=None, lo=None,
               exps=None):
    """Split FP32 / bf16 ``x [rows, cols]`` into 16-bit hi (+ lo) parts with per-row power-of-two exponents,
    or unpack INT16 ``x`` into its Dual-FP16 halves.  Returns (hi, lo or None, exps or None); parts come
    back as int16 tensors holding the 16-bit patterns (view them as float16 / bfloat16 as needed)."""
    import torch

    L = load()
    rows, cols = x.shape
    if x.dtype == torch.float32:
        xt = HEAL_F32
    elif x.dtype == torch.bfloat16:
        xt = HEAL_BF16
    elif x.dtype == torch.int16:
        xt, prescale, residual, part = HEAL_I16, False, True, "f16"
    else:
        raise TypeError(f"heal_split: unsupported dtype {x.dtype}")
    ld_part = (cols + 7) // 8 * 8
    if hi is None:
        hi = torch.empty((rows, ld_part), dtype=torch.int16, device=x.device)[:, :cols]
    if residual and lo is None:
        lo = torch.empty((rows, ld_part), dtype=torch.int16, device=x.device)[:, :cols]
    if prescale and exps is None:
        exps = torch.empty((rows,), dtype=torch.int32, device=x.device)
    lo_arg = lo if residual else None
    ex_arg = exps if prescale else None
    _check(L.heal_split(_ptr(x), xt, rows, cols, _ld(x), _PARTS[part], _ptr(hi), _ptr(lo_arg),
                        _ld(hi), _ptr(ex_arg), _stream(x.device)))
    return hi, lo_arg, ex_arg


def heal_unpack_i16(x, dual_split: str = "byte", hi=None, lo=None):
    """Dual-FP16 unpack of INT16 ``x [rows, cols]`` under the reading ``dual_split`` ("byte", "shift10" or
    "float"); returns (hi, lo) as int16 tensors holding the FP16 bit patterns."""
    import torch

    if x.dtype != torch.int16:
        raise TypeError("heal_unpack_i16: x must be int16")
    rows, cols = x.shape
    ld_part = (cols + 7) // 8 * 8
    if hi is None:
        hi = torch.empty((rows, ld_part), dtype=torch.int16, device=x.device)[:, :cols]
    if lo is None:
        lo = torch.empty((rows, ld_part), dtype=torch.int16, device=x.device)[:, :cols]
    _check(load().heal_unpack_i16(_ptr(x), rows, cols, _ld(x), _DUAL[dual_split], _ptr(hi), _ptr(lo), _ld(hi),
                                  _stream(x.device)))
    return hi, lo


def heal_channel_exponents(x, threshold_log2: int, col_exps=None):
    """Outlier-channel exponents of a calibration batch ``x [rows, cols]`` fp32: int32 [cols] with
    threshold_log2 - ilogb(max_r |x[r, c]|) for the columns whose maximum exceeds 2^threshold_log2, else 0."""
    import torch

    L = load()
    rows, cols = x.shape
    if col_exps is None:
        col_exps = torch.empty((cols,), dtype=torch.int32, device=x.device)
    _check(L.heal_channel_exponents(_ptr(x), rows, cols, _ld(x), int(threshold_log2), _ptr(col_exps),
                                    _stream(x.device)))
    return col_exps


def heal_split_scaled(x, col_exps, col_sign: int, part: str = "f16", prescale: bool = True,
                      residual: bool = True, hi=None, lo=None, exps=None):
    """heal_split of x' = x * 2^(col_sign * col_exps[c]) per column (col_sign +1 for activations, -1 for
    weights).  Returns (hi, lo or None, exps or None) like heal_split."""
    import torch

    L = load()
    rows, cols = x.shape
    if x.dtype == torch.float32:
        xt = HEAL_F32
    elif x.dtype == torch.bfloat16:
        xt = HEAL_BF16
    else:
        raise TypeError(f"heal_split_scaled: unsupported dtype {x.dtype}")
    ld_part = (cols + 7) // 8 * 8
    if hi is None:
        hi = torch.empty((rows, ld_part), dtype=torch.int16, device=x.device)[:, :cols]
    if residual and lo is None:
        lo = torch.empty((rows, ld_part), dtype=torch.int16, device=x.device)[:, :cols]
    if prescale and exps is None:
        exps = torch.empty((rows,), dtype=torch.int32, device=x.device)
    lo_arg = lo if residual else None
    ex_arg = exps if prescale else None
    _check(L.heal_split_scaled(_ptr(x), xt, rows, cols, _ld(x), _PARTS[part], _ptr(hi), _ptr(lo_arg), _ld(hi),
                               _ptr(ex_arg), _ptr(col_exps), int(col_sign), _stream(x.device)))
    return hi, lo_arg, ex_arg


# ---------------------------------------------------------------------------------------------- heal_gemm_comp
def heal_gemm_comp(a_hi, a_lo, a_exp, b_hi, b_lo, b_exp, part: str = "f16", c=None):
    """C [M, N] fp32 = sum of the 16-bit products of A's and B^T's parts, scaled by 2^-(ea_i + eb_j).
    ``a_*`` are [M, K] and ``b_*`` are parts of B^T [N, K] (both K-contiguous); lo / exp may be None."""
    import torch

    L = load()
    M, K = a_hi.shape
    N = b_hi.shape[0]
    if c is None:
        ldc = (N + 3) // 4 * 4
        c = torch.empty((M, ldc), dtype=torch.float32, device=a_hi.device)[:, :N]
    if a_lo is not None and (a_lo.shape != a_hi.shape or a_lo.stride() != a_hi.stride()):
        raise ValueError("a_lo must match a_hi's shape and strides")
    if b_lo is not None and (b_lo.shape != b_hi.shape or b_lo.stride() != b_hi.stride()):
        raise ValueError("b_lo must match b_hi's shape and strides")
    _check(L.heal_gemm_comp(M, N, K, _ptr(a_hi), _ptr(a_lo), _ptr(a_exp), _ld(a_hi), _ptr(b_hi), _ptr(b_lo),
                            _ptr(b_exp), _ld(b_hi), _PARTS[part], _ptr(c), _ld(c), _stream(a_hi.device)))
    return c


def heal_gemm_comp_workspace_bytes(M: int, N: int, K: int, products: int) -> int:
    """Workspace bytes heal_gemm_comp_splitk needs (0 when it does not split K)."""
    return int(load().heal_gemm_comp_workspace_bytes(M, N, K, products))


def heal_gemm_comp_splitk_slices(M: int, N: int, K: int, products: int) -> int:
    """K slices heal_gemm_comp_splitk uses (1: no split, the call is heal_gemm_comp)."""
    return int(load().heal_gemm_comp_splitk_slices(M, N, K, products))


def heal_gemm_comp_splitk(a_hi, a_lo, a_exp, b_hi, b_lo, b_exp, part: str = "f16", c=None, workspace=None):
    """heal_gemm_comp with K split across workgroups where its own launch would leave CUs idle (partials added
    in slice order).  A workspace of heal_gemm_comp_workspace_bytes() is allocated with torch when none is
    given."""
    import torch

    L = load()
    M, K = a_hi.shape
    N = b_hi.shape[0]
    if c is None:
        ldc = (N + 3) // 4 * 4
        c = torch.empty((M, ldc), dtype=torch.float32, device=a_hi.device)[:, :N]
    if a_lo is not None and (a_lo.shape != a_hi.shape or a_lo.stride() != a_hi.stride()):
        raise ValueError("a_lo must match a_hi's shape and strides")
    if b_lo is not None and (b_lo.shape != b_hi.shape or b_lo.stride() != b_hi.stride()):
        raise ValueError("b_lo must match b_hi's shape and strides")
    products = 1 + (a_lo is not None) + (b_lo is not None)
    ws_ptr, ws_bytes = None, 0
    if workspace is None:
        # products = 2 is sized as A's low part; B's low part alone plans like three products: cover both
        need = heal_gemm_comp_workspace_bytes(M, N, K, products)
        if products == 2:
            need = max(need, heal_gemm_comp_workspace_bytes(M, N, K, 3))
        if need:
            workspace = torch.empty((need + 255) // 256 * 256, dtype=torch.uint8, device=a_hi.device)
    if workspace is not None:
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    _check(L.heal_gemm_comp_splitk(M, N, K, _ptr(a_hi), _ptr(a_lo), _ptr(a_exp), _ld(a_hi), _ptr(b_hi), _ptr(b_lo),
                                   _ptr(b_exp), _ld(b_hi), _PARTS[part], _ptr(c), _ld(c), ws_ptr, ws_bytes,
                                   _stream(a_hi.device)))
    return c


def heal_row_exponents(x, exps=None):
    """Row exponents e = 14 - ilogb(max |x[r, :]|) of FP32 ``x [rows, cols]`` (those heal_split writes)."""
    import torch

    rows, cols = x.shape
    if exps is None:
        exps = torch.empty((rows,), dtype=torch.int32, device=x.device)
    _check(load().heal_row_exponents(_ptr(x), rows, cols, _ld(x), _ptr(exps), _stream(x.device)))
    return exps


def heal_gemm_comp_f32a(a, a_exp, b_hi, b_lo, b_exp, c=None):
    """Compensated GEMM with FP32 ``a [M, K]`` split inside the kernel (row exponents ``a_exp`` from
    heal_row_exponents, or None for M <= 16: the kernel derives the same ones) against FP16 parts of B^T
    ``[N, K]``; returns C [M, N] fp32, bit for bit what heal_split + heal_gemm_comp give."""
    import torch

    M, K = a.shape
    N = b_hi.shape[0]
    if c is None:
        c = torch.empty((M, (N + 3) // 4 * 4), dtype=torch.float32, device=a.device)[:, :N]
    if b_lo is not None and (b_lo.shape != b_hi.shape or b_lo.stride() != b_hi.stride()):
        raise ValueError("b_lo must match b_hi's shape and strides")
    _check(load().heal_gemm_comp_f32a(M, N, K, _ptr(a), _ld(a), _ptr(a_exp), _ptr(b_hi), _ptr(b_lo), _ptr(b_exp),
                                      _ld(b_hi), _ptr(c), _ld(c), _stream(a.device)))
    return c


def heal_gemm_comp_f32a_workspace_bytes(M: int, N: int, K: int, products: int) -> int:
    """Workspace bytes heal_gemm_comp_f32a_splitk needs with row exponents given (0 when it does not split K)."""
    return int(load().heal_gemm_comp_f32a_workspace_bytes(M, N, K, products))


def heal_gemm_comp_f32a_splitk_slices(M: int, N: int, K: int, products: int) -> int:
    """K slices heal_gemm_comp_f32a_splitk uses with row exponents given (1: no split)."""
    return int(load().heal_gemm_comp_f32a_splitk_slices(M, N, K, products))


def heal_gemm_comp_f32a_splitk(a, a_exp, b_hi, b_lo, b_exp, c=None, workspace=None):
    """heal_gemm_comp_f32a with K split across workgroups for 8..16 rows and K >= 8192 (row exponents ``a_exp``
    required for the split; partials added in slice order): bit for bit heal_split + heal_gemm_comp_splitk.  A
    workspace of heal_gemm_comp_f32a_workspace_bytes() is allocated with torch when none is given."""
    import torch

    L = load()
    M, K = a.shape
    N = b_hi.shape[0]
    if c is None:
        c = torch.empty((M, (N + 3) // 4 * 4), dtype=torch.float32, device=a.device)[:, :N]
    if b_lo is not None and (b_lo.shape != b_hi.shape or b_lo.stride() != b_hi.stride()):
        raise ValueError("b_lo must match b_hi's shape and strides")
    ws_ptr, ws_bytes = None, 0
    if workspace is None and a_exp is not None:
        need = heal_gemm_comp_f32a_workspace_bytes(M, N, K, 3 if b_lo is not None else 2)
        if need:
            workspace = torch.empty((need + 255) // 256 * 256, dtype=torch.uint8, device=a.device)
    if workspace is not None:
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    _check(L.heal_gemm_comp_f32a_splitk(M, N, K, _ptr(a), _ld(a), _ptr(a_exp), _ptr(b_hi), _ptr(b_lo), _ptr(b_exp),
                                        _ld(b_hi), _ptr(c), _ld(c), ws_ptr, ws_bytes, _stream(a.device)))
    return c


def heal_gemm_comp_quant_i16(a_hi, a_lo, a_exp, b_hi, b_lo, b_exp, q=None, scale=None):
    """The compensated GEMM with INT16 quantisation per (row, 128-column head) in its epilogue.  Returns
    (q int16 [M, N], scale fp32 [M, N / 128]); ``q`` / ``scale`` may be row-strided views into a cache."""
    import torch

    L = load()
    M, K = a_hi.shape
    N = b_hi.shape[0]
    if q is None:
        q = torch.empty((M, N), dtype=torch.int16, device=a_hi.device)
    if scale is None:
        scale = torch.empty((M, N // 128), dtype=torch.float32, device=a_hi.device)
    if a_lo is not None and (a_lo.shape != a_hi.shape or a_lo.stride() != a_hi.stride()):
        raise ValueError("a_lo must match a_hi's shape and strides")
    if b_lo is not None and (b_lo.shape != b_hi.shape or b_lo.stride() != b_hi.stride()):
        raise ValueError("b_lo must match b_hi's shape and strides")
    _check(L.heal_gemm_comp_quant_i16(M, N, K, _ptr(a_hi), _ptr(a_lo), _ptr(a_exp), _ld(a_hi), _ptr(b_hi),
                                      _ptr(b_lo), _ptr(b_exp), _ld(b_hi), _PARTS["f16"], _ptr(q), _ld(q),
                                      _ptr(scale), _ld(scale), _stream(a_hi.device)))
    return q, scale


def heal_gemm_comp_variant(M: int, N: int, K: int, products: int) -> str:
    """Name of the kernel instantiation heal_gemm_comp launches for this shape and product count."""
    return load().heal_gemm_comp_variant(M, N, K, products).decode()


# ------------------------------------------------------------------------------------------ heal_qkv_quant_i16
def heal_qkv_quant_i16(x, q=None, scale=None):
    """INT16-quantise fp32 ``x [tokens, heads, head_dim]`` per (token, head).  Returns (q int16, scale fp32).
    ``q`` / ``scale`` may be views into a larger cache ([tokens, heads, head_dim] with any token stride)."""
    import torch

    L = load()
    T, H, D = x.shape
    if x.stride(2) != 1 or x.stride(1) != D:
        raise ValueError("x must have heads packed at stride head_dim and a contiguous last axis")
    if q is None:
        q = torch.empty((T, H, D), dtype=torch.int16, device=x.device)
    if scale is None:
        scale = torch.empty((T, H), dtype=torch.float32, device=x.device)
    if q.stride(2) != 1 or q.stride(1) != D or scale.stride(1) != 1:
        raise ValueError("q / scale must have heads packed")
    _check(L.heal_qkv_quant_i16(_ptr(x), T, H, D, x.stride(0), _ptr(q), q.stride(0), _ptr(scale),
                                scale.stride(0), _stream(x.device)))
    return q, scale


# ----------------------------------------------------------------------------------------- heal_attn_dual_fp16
def make_attn_args(q, q_scale, k, k_scale, v, v_scale, out, causal: bool = True,
                   softmax_scale: float | None = None, workspace=None, dual_split: str = "byte") -> HealAttnArgs:
    """Fill heal_attn_args from torch tensors q [B, Lq, Hq, D], k/v [B, Lkv, Hkv, D] (int16), scales
    [B, L, H] (fp32) and out [B, Lq, Hq, D] (fp32).  k and v must share strides, as must their scales."""
    B, Lq, Hq, D = q.shape
    Lkv, Hkv = k.shape[1], k.shape[2]
    if k.stride() != v.stride() or k_scale.stride() != v_scale.stride():
        raise ValueError("k and v (and their scales) must share strides")
    for t in (q, k, v, out):
        if t.stride(3) != 1:
            raise ValueError("head_dim axis must be contiguous")
    a = HealAttnArgs()
    a.batch, a.q_len, a.kv_len, a.n_q_heads, a.n_kv_heads, a.head_dim = B, Lq, Lkv, Hq, Hkv, D
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.q_scale, a.k_scale, a.v_scale = q_scale.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr()
    a.q_strides[:] = list(q.stride()[:3])
    a.kv_strides[:] = list(k.stride()[:3])
    a.qs_strides[:] = list(q_scale.stride()[:3])
    a.kvs_strides[:] = list(k_scale.stride()[:3])
    a.o_strides[:] = list(out.stride()[:3])
    a.causal = 1 if causal else 0
    a.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    a.dual_split = _DUAL[dual_split]
    a.out = out.data_ptr()
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def heal_attn_workspace_bytes(args: HealAttnArgs) -> int:
    return int(load().heal_attn_workspace_bytes(ctypes.byref(args)))


def heal_attn_dual_fp16(q, q_scale, k, k_scale, v, v_scale, causal: bool = True,
                        softmax_scale: float | None = None, out=None, workspace=None, dual_split: str = "byte"):
    """Attention over INT16 Q/K/V with Dual-FP16 products and FP32 softmax; returns out [B, Lq, Hq, D] fp32.
    ``dual_split`` selects the reading of the pair ("byte", "shift10" or "float").  A workspace of
    heal_attn_workspace_bytes() is allocated with torch when none is given."""
    import torch

    L = load()
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    args = make_attn_args(q, q_scale, k, k_scale, v, v_scale, out, causal, softmax_scale, workspace, dual_split)
    need = heal_attn_workspace_bytes(args)
    if need and workspace is None:
        workspace = torch.empty((need + 255) // 256 * 256, dtype=torch.uint8, device=q.device)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel()
    _check(L.heal_attn_dual_fp16(ctypes.byref(args), _stream(q.device)))
    return out


def heal_attn_dual_fp16_noalloc(q, q_scale, k, k_scale, v, v_scale, out, causal: bool = True,
                                softmax_scale: float | None = None, dual_split: str = "byte"):
    """heal_attn_dual_fp16 into the caller's ``out`` without any workspace: the library keeps the decode
    partials in its own device scratch (calls that overlap on one GPU race on it)."""
    args = make_attn_args(q, q_scale, k, k_scale, v, v_scale, out, causal, softmax_scale, None, dual_split)
    _check(load().heal_attn_dual_fp16_noalloc(ctypes.byref(args), _stream(q.device)))
    return out


def make_paged_args(q, q_scale, k_pages, k_scale, v_pages, v_scale, block_table, seq_lens, max_kv_len: int,
                    out, softmax_scale: float | None = None, workspace=None,
                    dual_split: str = "byte") -> HealPagedDecodeArgs:
    """Fill heal_paged_decode_args from torch tensors: q [B, Hq, D] int16, q_scale [B, Hq] fp32, k/v pages
    [P, page_size, Hkv, D] int16, their scales [P, page_size, Hkv] fp32, block_table [B, max_pages] int32,
    seq_lens [B] int32 and out [B, Hq, D] fp32.  k and v pages (and their scales) must share strides."""
    B, Hq, D = q.shape
    P, ps, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if k_pages.stride() != v_pages.stride() or k_scale.stride() != v_scale.stride():
        raise ValueError("k and v pages (and their scales) must share strides")
    for t in (q, k_pages, v_pages, out):
        if t.stride(-1) != 1:
            raise ValueError("head_dim axis must be contiguous")
    a = HealPagedDecodeArgs()
    a.batch, a.n_q_heads, a.n_kv_heads, a.head_dim = B, Hq, Hkv, D
    a.page_size, a.num_pages, a.max_pages_per_seq, a.max_kv_len = ps, P, block_table.shape[1], int(max_kv_len)
    a.q, a.q_scale = q.data_ptr(), q_scale.data_ptr()
    a.k_pages, a.v_pages = k_pages.data_ptr(), v_pages.data_ptr()
    a.k_scale, a.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
    a.block_table, a.seq_lens = block_table.data_ptr(), seq_lens.data_ptr()
    a.q_strides[:] = list(q.stride()[:2])
    a.qs_strides[:] = list(q_scale.stride()[:2])
    a.kv_strides[:] = list(k_pages.stride()[:3])
    a.kvs_strides[:] = list(k_scale.stride()[:3])
    a.o_strides[:] = list(out.stride()[:2])
    a.bt_stride = block_table.stride(0)
    a.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    a.dual_split = _DUAL[dual_split]
    a.out = out.data_ptr()
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a


def heal_attn_paged_workspace_bytes(args: HealPagedDecodeArgs) -> int:
    return int(load().heal_attn_paged_workspace_bytes(ctypes.byref(args)))


def heal_attn_decode_paged(q, q_scale, k_pages, k_scale, v_pages, v_scale, block_table, seq_lens,
                           max_kv_len: int, softmax_scale: float | None = None, out=None, workspace=None,
                           dual_split: str = "byte"):
    """Decode attention (one query token per sequence) over a paged INT16 KV cache; returns out [B, Hq, D]
    fp32.  A workspace of heal_attn_paged_workspace_bytes() is allocated with torch when none is given."""
    import torch

    L = load()
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    args = make_paged_args(q, q_scale, k_pages, k_scale, v_pages, v_scale, block_table, seq_lens, max_kv_len,
                           out, softmax_scale, workspace, dual_split)
    need = heal_attn_paged_workspace_bytes(args)
    if need and workspace is None:
        workspace = torch.empty((need + 255) // 256 * 256, dtype=torch.uint8, device=q.device)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel()
    _check(L.heal_attn_decode_paged(ctypes.byref(args), _stream(q.device)))
    return out
