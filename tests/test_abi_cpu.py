"""The C ABI on the CPU: libheal.so loads, exports every entry point include/heal.h declares, the
ctypes mirror of heal_attn_args matches the C layout, and every validation error is returned before any
device work (so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "heal.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"HEAL_API\s+[\w\s\*]+?\b(heal_\w+)\s*\(", txt)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("heal_split", "heal_gemm_comp", "heal_qkv_quant_i16", "heal_attn_dual_fp16",
              "heal_attn_workspace_bytes", "heal_status_str", "heal_abi_version", "heal_attn_decode_paged",
              "heal_attn_paged_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(heal):
    lib = heal.load()
    for n in _declared():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", heal.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (heal_\w+)$", out, re.M))
    assert set(_declared()) <= exported
    # nothing else leaks out of the library's namespace
    assert all(s.startswith("heal_") for s in exported)


def test_glue_library_exports_every_declared_symbol():
    """the decoder-block glue of the model-level check (include/heal_glue.h, libheal_glue.so)"""
    txt = open(os.path.join(ROOT, "include", "heal_glue.h")).read()
    names = sorted(set(re.findall(r"GLUE_API\s+int\s+(glue_\w+)\s*\(", txt)))
    assert len(names) == 7
    lib_path = os.path.join(ROOT, "error_compensated_gemm_amd", "libheal_glue.so")
    lib = ctypes.CDLL(lib_path)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True, text=True).stdout
    assert set(names) == set(re.findall(r" T (glue_\w+)$", out, re.M))


def test_glue_grid_limits_refused_before_launch():
    """glue calls whose grid would pass 2^32 work-items per dimension return 6 before any runtime call"""
    lib = ctypes.CDLL(os.path.join(ROOT, "error_compensated_gemm_amd", "libheal_glue.so"))
    for f in (lib.glue_embed, lib.glue_rmsnorm, lib.glue_rope, lib.glue_swiglu, lib.glue_add, lib.glue_argmax,
              lib.glue_add_rmsnorm):
        f.restype = ctypes.c_int
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    fake = vp(FAKE)
    assert lib.glue_embed(fake, fake, i64(1 << 24), i64(128), fake, None) == 6
    assert lib.glue_rmsnorm(fake, i64(1 << 24), i64(128), ctypes.c_float(1e-5), fake, None) == 6
    assert lib.glue_add_rmsnorm(fake, fake, i64(1 << 24), i64(128), ctypes.c_float(1e-5), fake, None) == 6
    assert lib.glue_rope(fake, i64(1 << 26), i64(1), i64(128), i64(0), fake, None) == 6
    assert lib.glue_rope(fake, i64(1), i64(1 << 32), i64(128), i64(0), fake, None) == 6
    assert lib.glue_swiglu(fake, fake, i64(1 << 32), fake, None) == 6
    assert lib.glue_add(fake, fake, i64(1 << 32), None) == 6
    assert lib.glue_argmax(fake, i64(1 << 31), fake, None) == 6
    assert lib.glue_add(fake, fake, i64(0), None) == 0  # empty: nothing to do


def test_version_and_status_strings(heal):
    lib = heal.load()
    assert lib.heal_abi_version() == 7
    for s in range(9):
        assert lib.heal_status_str(s).decode().startswith("HEAL")
    assert b"unknown" in lib.heal_status_str(99)


@pytest.mark.parametrize("cname,pyname", [("heal_attn_args", "HealAttnArgs"),
                                          ("heal_paged_decode_args", "HealPagedDecodeArgs")])
def test_args_layout_matches_c(heal, tmp_path, cname, pyname):
    cls = getattr(heal, pyname)
    fields = [f for f, _ in cls._fields_]
    src = tmp_path / "layout.c"
    body = "".join(f'  printf("{f} %zu\\n", offsetof({cname}, {f}));\n' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "heal.h"\nint main(void) {\n'
                   f'  printf("size %zu\\n", sizeof({cname}));\n{body}  return 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split("\n")
               if line)
    assert int(got["size"]) == ctypes.sizeof(cls)
    for f in fields:
        assert int(got[f]) == getattr(cls, f).offset, f


P = ctypes.c_void_p
FAKE = 0x100000  # 16-byte aligned, never dereferenced: each call below fails validation first
MIS = FAKE + 2


def test_split_validation(heal):
    lib = heal.load()
    F32, BF16, F16, I16 = 0, 1, 2, 3
    assert lib.heal_split(None, F32, 4, 8, 8, F16, P(FAKE), P(FAKE), 8, P(FAKE), None) == 1   # NULL x
    assert lib.heal_split(P(FAKE), F32, -1, 8, 8, F16, P(FAKE), None, 8, None, None) == 2     # shape
    assert lib.heal_split(P(FAKE), F32, 4, 8, 4, F16, P(FAKE), None, 8, None, None) == 3      # ld_x < cols
    assert lib.heal_split(P(MIS), F32, 4, 8, 8, F16, P(FAKE), None, 8, None, None) == 4       # f32 misaligned
    assert lib.heal_split(P(FAKE), F32, 4, 8, 8, F16, P(MIS), None, 8, None, None) == 4       # parts misaligned
    assert lib.heal_split(P(FAKE), F32, 4, 8, 8, F16, P(FAKE), None, 12, None, None) == 4     # ld_part % 8
    assert lib.heal_split(P(FAKE), 7, 4, 8, 8, F16, P(FAKE), None, 8, None, None) == 5        # x dtype
    assert lib.heal_split(P(FAKE), F32, 4, 8, 8, F32, P(FAKE), None, 8, None, None) == 5      # part dtype
    assert lib.heal_split(P(FAKE), I16, 4, 8, 8, F16, P(FAKE), P(FAKE), 8, P(FAKE), None) == 5  # I16 + exps
    assert lib.heal_split(P(FAKE), I16, 4, 8, 8, F16, P(FAKE), None, 8, None, None) == 1      # I16 needs lo
    assert lib.heal_split(None, F32, 0, 8, 8, F16, None, None, 8, None, None) == 0            # empty: OK


def test_unpack_validation(heal):
    lib = heal.load()
    un = lib.heal_unpack_i16
    assert un(None, 4, 8, 8, 0, P(FAKE), P(FAKE), 8, None) == 1       # NULL x
    assert un(P(FAKE), 4, 8, 8, 0, P(FAKE), None, 8, None) == 1       # NULL lo
    assert un(P(FAKE), 4, -8, 8, 0, P(FAKE), P(FAKE), 8, None) == 2   # shape
    assert un(P(FAKE), 4, 8, 8, 3, P(FAKE), P(FAKE), 8, None) == 5    # unknown reading
    assert un(P(FAKE), 4, 8, 4, 1, P(FAKE), P(FAKE), 8, None) == 3    # ld_x < cols
    assert un(P(FAKE + 1), 4, 8, 8, 2, P(FAKE), P(FAKE), 8, None) == 4  # x not int16-aligned
    assert un(P(FAKE), 4, 8, 8, 2, P(MIS), P(FAKE), 8, None) == 4     # hi misaligned
    assert un(P(FAKE), 4, 8, 8, 2, P(FAKE), P(FAKE), 12, None) == 4   # ld_part % 8
    assert un(P(FAKE), 0, 8, 8, 2, P(FAKE), P(FAKE), 8, None) == 0    # empty: no launch


def test_row_exponents_and_f32a_validation(heal):
    lib = heal.load()
    rx = lib.heal_row_exponents
    assert rx(P(FAKE), 4, 8, 8, None, None) == 1          # NULL exps
    assert rx(None, 4, 8, 8, P(FAKE), None) == 1          # NULL x with columns
    assert rx(P(FAKE), -1, 8, 8, P(FAKE), None) == 2
    assert rx(P(FAKE), 4, 8, 7, P(FAKE), None) == 3       # ld_x < cols
    assert rx(P(FAKE + 2), 4, 8, 8, P(FAKE), None) == 4   # x not 4-byte aligned
    assert rx(P(FAKE), 0, 8, 8, None, None) == 0          # no rows: nothing to do
    g = lib.heal_gemm_comp_f32a
    ok = dict(M=64, N=32, K=100, a=P(FAKE), lda=100, ae=P(FAKE), bh=P(FAKE), bl=None, be=None, ldb=104,
              c=P(FAKE), ldc=32)
    call = lambda **kw: g(*[{**ok, **kw}[k] for k in ("M", "N", "K", "a", "lda", "ae", "bh", "bl", "be", "ldb",
                                                       "c", "ldc")], None)
    assert call(K=-1) == 2
    assert call(ae=None) == 1                             # the row exponents are required above 16 rows
    assert call(M=17, ae=None) == 1
    assert call(M=16, ae=None, a=P(FAKE + 4)) == 4        # 16 rows may omit them; the other checks still apply
    assert call(a=None) == 1 and call(c=None) == 1 and call(bh=None) == 1
    assert call(lda=96) == 3 and call(ldb=96) == 3 and call(ldc=16) == 3
    assert call(a=P(FAKE + 4)) == 4                       # a not 16-byte aligned
    assert call(lda=102) == 4                             # lda not a multiple of 4
    assert call(ldb=100) == 4                             # ldb not a multiple of 8
    assert call(M=0) == 0


def test_gemm_validation(heal):
    lib = heal.load()
    F16, F32 = 2, 0
    ok = dict(M=4, N=4, K=8)
    args = lambda M=4, N=4, K=8, ah=FAKE, bh=FAKE, c=FAKE, lda=8, ldb=8, ldc=4, part=F16, al=None: (
        M, N, K, P(ah) if ah else None, P(al) if al else None, None, lda, P(bh) if bh else None, None, None,
        ldb, part, P(c) if c else None, ldc, None)
    assert lib.heal_gemm_comp(*args(M=-1)) == 2
    assert lib.heal_gemm_comp(*args(ah=None)) == 1
    assert lib.heal_gemm_comp(*args(c=None)) == 1
    assert lib.heal_gemm_comp(*args(lda=4)) == 3
    assert lib.heal_gemm_comp(*args(ldc=2)) == 3
    assert lib.heal_gemm_comp(*args(ah=MIS)) == 4
    assert lib.heal_gemm_comp(*args(al=MIS)) == 4
    assert lib.heal_gemm_comp(*args(ldb=12)) == 4
    assert lib.heal_gemm_comp(*args(ldc=6)) == 4
    assert lib.heal_gemm_comp(*args(part=F32)) == 5
    assert lib.heal_gemm_comp(*args(M=0)) == 0


def test_quant_validation(heal):
    lib = heal.load()
    assert lib.heal_qkv_quant_i16(P(FAKE), 4, 2, 130, 512, P(FAKE), 512, P(FAKE), 2, None) == 6  # head_dim % 4
    assert lib.heal_qkv_quant_i16(P(FAKE), 4, 2, 2048, 4096, P(FAKE), 4096, P(FAKE), 2, None) == 6
    assert lib.heal_qkv_quant_i16(None, 4, 2, 128, 256, P(FAKE), 256, P(FAKE), 2, None) == 1
    assert lib.heal_qkv_quant_i16(P(FAKE), 4, 2, 128, 128, P(FAKE), 256, P(FAKE), 2, None) == 3
    assert lib.heal_qkv_quant_i16(P(FAKE), 4, 2, 128, 256, P(FAKE), 256, P(FAKE), 1, None) == 3
    assert lib.heal_qkv_quant_i16(P(MIS), 4, 2, 128, 256, P(FAKE), 256, P(FAKE), 2, None) == 4
    assert lib.heal_qkv_quant_i16(P(FAKE), 4, 2, 128, 258, P(FAKE), 256, P(FAKE), 2, None) == 4
    assert lib.heal_qkv_quant_i16(P(FAKE), -4, 2, 128, 256, P(FAKE), 256, P(FAKE), 2, None) == 2
    assert lib.heal_qkv_quant_i16(P(FAKE), 0, 2, 128, 256, P(FAKE), 256, P(FAKE), 2, None) == 0


def _attn_args(heal, **kw):
    a = heal.HealAttnArgs()
    a.batch, a.q_len, a.kv_len, a.n_q_heads, a.n_kv_heads, a.head_dim = 1, 4, 4, 2, 1, 128
    a.q = a.k = a.v = a.out = FAKE
    a.q_scale = a.k_scale = a.v_scale = FAKE
    a.q_strides[:] = [4 * 2 * 128, 2 * 128, 128]
    a.kv_strides[:] = [4 * 128, 128, 128]
    a.qs_strides[:] = [8, 2, 1]
    a.kvs_strides[:] = [4, 1, 1]
    a.o_strides[:] = [4 * 2 * 128, 2 * 128, 128]
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_attn_validation(heal):
    lib = heal.load()
    call = lambda **kw: lib.heal_attn_dual_fp16(ctypes.byref(_attn_args(heal, **kw)), None)
    assert lib.heal_attn_dual_fp16(None, None) == 1
    assert call(head_dim=64) == 6
    assert call(n_q_heads=3, n_kv_heads=2) == 2
    assert call(batch=-1) == 2
    assert call(q=0) == 1
    assert call(k=0) == 1
    assert call(out=MIS) == 4
    assert call(softmax_scale=-1.0) == 2
    assert call(dual_split=3) == 5 and call(dual_split=-1) == 5  # not a reading of the Dual-FP16 pair
    a = _attn_args(heal)
    a.q_strides[1] = 100  # not a multiple of 8
    assert lib.heal_attn_dual_fp16(ctypes.byref(a), None) == 4
    a = _attn_args(heal)
    a.kv_strides[2] = 64  # smaller than head_dim
    assert lib.heal_attn_dual_fp16(ctypes.byref(a), None) == 3
    # decode needs a workspace: none given -> HEAL_ERR_WORKSPACE before any launch
    a = _attn_args(heal, q_len=1, kv_len=5000)
    assert lib.heal_attn_workspace_bytes(ctypes.byref(a)) > 0
    assert lib.heal_attn_dual_fp16(ctypes.byref(a), None) == 8
    a = _attn_args(heal, q_len=1, kv_len=5000, workspace=FAKE, workspace_bytes=16)
    assert lib.heal_attn_dual_fp16(ctypes.byref(a), None) == 8
    assert call(batch=0) == 0


def test_attn_noalloc_validation(heal):
    """heal_attn_dual_fp16_noalloc applies heal_attn_dual_fp16's checks and refuses, on the host before any
    device call, a decode whose partials would not fit the library's fixed scratch."""
    lib = heal.load()
    call = lambda **kw: lib.heal_attn_dual_fp16_noalloc(ctypes.byref(_attn_args(heal, **kw)), None)
    assert lib.heal_attn_dual_fp16_noalloc(None, None) == 1
    assert call(head_dim=64) == 6
    assert call(n_q_heads=3, n_kv_heads=2) == 2
    assert call(out=MIS) == 4
    assert call(dual_split=3) == 5
    assert call(batch=0) == 0
    # 64 x 20000 keys, 32 / 8 heads: 64 * 32 * 10 partials of 528 bytes, over the 8 MiB scratch
    big = dict(batch=64, q_len=1, kv_len=20000, n_q_heads=32, n_kv_heads=8)
    a = _attn_args(heal, **big)
    assert lib.heal_attn_workspace_bytes(ctypes.byref(a)) > heal.HEAL_ATTN_NOALLOC_MAX_WORKSPACE
    assert lib.heal_attn_dual_fp16_noalloc(ctypes.byref(a), None) == 8


def test_grid_limits_refused_before_launch(heal):
    """Shapes whose launch grid would pass HIP's 2^32 work-items per dimension are refused with
    HEAL_ERR_UNSUPPORTED before any runtime call (a truncated grid would silently skip rows); sizes
    whose workspace product overflows 64 bits saturate instead of wrapping to a small number."""
    lib = heal.load()
    F32, F16 = 0, 2
    # split of 2^26 rows: 2^24 workgroups of 256 work-items
    assert lib.heal_split(P(FAKE), F32, 1 << 26, 1, 1, F16, P(FAKE), None, 8, None, None) == 6
    assert lib.heal_unpack_i16(P(FAKE), 1 << 26, 8, 8, 0, P(FAKE), P(FAKE), 8, None) == 6
    assert lib.heal_row_exponents(P(FAKE), 1 << 26, 1, 1, P(FAKE), None) == 6
    # quantiser over 2^33 (token, head) rows
    assert lib.heal_qkv_quant_i16(P(FAKE), 1 << 30, 8, 128, 1024, P(FAKE), 1024, P(FAKE), 8, None) == 6
    # GEMM: K above 2^31 is a shape error; a skinny GEMM 2^31 columns wide has too many workgroups
    big = (1 << 31) + 8
    assert lib.heal_gemm_comp(4, 4, big, P(FAKE), None, None, big, P(FAKE), None, None, big, F16, P(FAKE), 4,
                              None) == 2
    assert lib.heal_gemm_comp(16, 1 << 31, 8, P(FAKE), None, None, 8, P(FAKE), None, None, 8, F16, P(FAKE),
                              1 << 31, None) == 6
    # attention: 2^30 (batch, head) prefill workgroups; 2^33 (batch, kv-head) decode rows
    a = _attn_args(heal, batch=1 << 20, n_q_heads=1 << 10, n_kv_heads=1 << 10)
    assert lib.heal_attn_dual_fp16(ctypes.byref(a), None) == 6
    a = _attn_args(heal, batch=1 << 24, n_q_heads=1 << 9, n_kv_heads=1 << 9, q_len=1, kv_len=5000)
    need = lib.heal_attn_workspace_bytes(ctypes.byref(a))
    assert need == (1 << 24) * (1 << 9) * 3 * (4 + 128) * 4
    a.workspace, a.workspace_bytes = FAKE, need
    assert lib.heal_attn_dual_fp16(ctypes.byref(a), None) == 6
    a = _attn_args(heal, batch=1 << 40, n_q_heads=1 << 30, n_kv_heads=1 << 30, q_len=1, kv_len=1)
    assert lib.heal_attn_workspace_bytes(ctypes.byref(a)) == (1 << 63) - 1


def test_splitk_validation_and_plan(heal):
    """heal_gemm_comp_splitk: heal_gemm_comp's checks, then the workspace (needed only where K is split)"""
    lib = heal.load()
    F16, F32 = 2, 0
    # 128 x 4096 x 14336 with A's low part splits K (32 tiles of 128 x 128); 2048 x 4096 x 4096 does not
    assert heal.heal_gemm_comp_splitk_slices(128, 4096, 14336, 2) == 8
    need = heal.heal_gemm_comp_workspace_bytes(128, 4096, 14336, 2)
    assert need == 8 * 128 * 4096 * 4
    assert heal.heal_gemm_comp_workspace_bytes(2048, 4096, 4096, 2) == 0
    assert heal.heal_gemm_comp_splitk_slices(2048, 4096, 4096, 2) == 1
    assert heal.heal_gemm_comp_splitk_slices(16, 4096, 14336, 2) == 11     # 16 rows, long K: slices of 1408
    assert heal.heal_gemm_comp_splitk_slices(16, 4096, 4096, 2) == 1       # 16-row skinny, K < 8192: whole
    assert heal.heal_gemm_comp_splitk_slices(4, 4096, 14336, 2) == 1       # under 8 rows: whole
    assert heal.heal_gemm_comp_splitk_slices(64, 4096, 14336, 2) == 8      # 64-row skinny: split
    assert heal.heal_gemm_comp_workspace_bytes(-1, 4, 4, 2) == 0 and heal.heal_gemm_comp_splitk_slices(4, 4, 4, 0) == 1
    # K per slice at least 1024 for tiles: 256 x 4096 x 1500 stays whole
    assert heal.heal_gemm_comp_splitk_slices(256, 4096, 1500, 2) == 1

    def call(M=128, N=4096, K=14336, ah=FAKE, al=FAKE, bh=FAKE, c=FAKE, lda=14336, ldb=14336, ldc=4096, part=F16,
             ws=FAKE, ws_bytes=need):
        return lib.heal_gemm_comp_splitk(M, N, K, P(ah) if ah else None, P(al) if al else None, None, lda,
                                         P(bh) if bh else None, None, None, ldb, part, P(c) if c else None, ldc,
                                         P(ws) if ws else None, ws_bytes, None)
    assert call(M=-1) == 2
    assert call(K=(1 << 31) + 8, lda=(1 << 31) + 8, ldb=(1 << 31) + 8) == 2
    assert call(part=F32) == 5
    assert call(ah=None) == 1 and call(c=None) == 1
    assert call(lda=100) == 3 and call(ldc=100) == 3
    assert call(ah=MIS) == 4 and call(ldc=4098) == 4
    assert call(ws=None) == 8                       # workspace needed, none given
    assert call(ws_bytes=need - 4) == 8             # too small
    assert call(ws=FAKE + 16) == 8                  # not 256-byte aligned
    assert call(M=0) == 0                           # empty: nothing to do


def test_f32a_splitk_validation_and_plan(heal):
    """heal_gemm_comp_f32a_splitk: heal_gemm_comp_f32a's checks, then the workspace, needed only where K is split:
    8..16 rows with K >= 8192 and row exponents given, the slices of heal_gemm_comp_splitk"""
    lib = heal.load()
    for M, N, K, P_ in ((16, 4096, 14336, 2), (16, 4096, 14336, 3), (8, 4096, 8192, 2), (13, 1000, 9001, 3)):
        assert heal.heal_gemm_comp_f32a_splitk_slices(M, N, K, P_) == heal.heal_gemm_comp_splitk_slices(M, N, K, P_)
        assert heal.heal_gemm_comp_f32a_workspace_bytes(M, N, K, P_) == heal.heal_gemm_comp_workspace_bytes(M, N, K, P_)
    assert heal.heal_gemm_comp_f32a_splitk_slices(16, 4096, 14336, 2) == 11  # slices of 1408 (A's parts in LDS)
    need = heal.heal_gemm_comp_f32a_workspace_bytes(16, 4096, 14336, 2)
    assert need == 11 * 16 * 4096 * 4
    assert heal.heal_gemm_comp_f32a_splitk_slices(16, 4096, 4096, 2) == 1     # K < 8192: whole
    assert heal.heal_gemm_comp_f32a_splitk_slices(4, 4096, 14336, 2) == 1     # under 8 rows: whole
    assert heal.heal_gemm_comp_f32a_splitk_slices(64, 4096, 14336, 2) == 1    # over 16 rows: whole (FP32 A)
    assert heal.heal_gemm_comp_f32a_splitk_slices(128, 4096, 14336, 2) == 1   # tile kernels: whole (FP32 A)
    assert heal.heal_gemm_comp_f32a_workspace_bytes(16, 4096, 14336, 1) == 0   # A always has its low part
    assert heal.heal_gemm_comp_f32a_splitk_slices(16, 4096, 14336, 4) == 1
    assert heal.heal_gemm_comp_f32a_workspace_bytes(-1, 4, 4, 2) == 0

    def call(M=16, N=4096, K=14336, a=FAKE, ea=FAKE, bh=FAKE, c=FAKE, lda=14336, ldb=14336, ldc=4096, ws=FAKE,
             ws_bytes=need):
        return lib.heal_gemm_comp_f32a_splitk(M, N, K, P(a) if a else None, lda, P(ea) if ea else None,
                                              P(bh) if bh else None, None, None, ldb, P(c) if c else None, ldc,
                                              P(ws) if ws else None, ws_bytes, None)
    assert call(M=-1) == 2
    assert call(K=(1 << 31) + 8, lda=(1 << 31) + 8, ldb=(1 << 31) + 8) == 2
    assert call(a=None) == 1 and call(c=None) == 1 and call(M=17, ea=None) == 1
    assert call(lda=100) == 3 and call(ldc=100) == 3
    assert call(a=MIS) == 4 and call(lda=14338) == 4 and call(ldc=4098) == 4
    assert call(ws=None) == 8                       # workspace needed, none given
    assert call(ws_bytes=need - 4) == 8             # too small
    assert call(ws=FAKE + 16) == 8                  # not 256-byte aligned
    assert call(M=0) == 0                           # empty: nothing to do


def test_gemm_variant_names(heal):
    assert heal.heal_gemm_comp_variant(0, 5, 5, 2) == "none"
    assert heal.heal_gemm_comp_variant(8192, 8192, 8192, 3).startswith("gemm_comp_kernel")
    assert heal.heal_gemm_comp_variant(8192, 8192, 8192, 3).endswith("P3")


def _paged_args(heal, **kw):
    a = heal.HealPagedDecodeArgs()
    a.batch, a.n_q_heads, a.n_kv_heads, a.head_dim = 2, 8, 2, 128
    a.page_size, a.num_pages, a.max_pages_per_seq, a.max_kv_len = 64, 10, 4, 256
    a.q = a.k_pages = a.v_pages = a.out = FAKE
    a.q_scale = a.k_scale = a.v_scale = a.block_table = a.seq_lens = FAKE
    a.q_strides[:] = [8 * 128, 128]
    a.qs_strides[:] = [8, 1]
    a.kv_strides[:] = [64 * 2 * 128, 2 * 128, 128]
    a.kvs_strides[:] = [64 * 2, 2, 1]
    a.o_strides[:] = [8 * 128, 128]
    a.bt_stride = 4
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_paged_decode_validation(heal):
    lib = heal.load()
    call = lambda **kw: lib.heal_attn_decode_paged(ctypes.byref(_paged_args(heal, **kw)), None)
    assert lib.heal_attn_decode_paged(None, None) == 1
    assert call(head_dim=64) == 6
    assert call(page_size=16) == 6      # below 32
    assert call(page_size=96) == 6      # not a power of two
    assert call(n_q_heads=34, n_kv_heads=2) == 6  # more than 16 query heads per kv head
    assert call(n_q_heads=9) == 2       # n_q_heads % n_kv_heads
    assert call(max_pages_per_seq=3) == 2   # 3 pages of 64 cannot hold 256 keys
    assert call(num_pages=0) == 2
    assert call(batch=-1) == 2
    assert call(seq_lens=0) == 1
    assert call(block_table=0) == 1
    assert call(k_pages=0) == 1
    assert call(bt_stride=3) == 3
    assert call(softmax_scale=float("inf")) == 2
    assert call(dual_split=7) == 5
    assert call(v_pages=MIS) == 4
    assert call(block_table=FAKE + 2) == 4
    a = _paged_args(heal)
    a.kv_strides[1] = 260  # not a multiple of 8
    assert lib.heal_attn_decode_paged(ctypes.byref(a), None) == 4
    a = _paged_args(heal)
    a.q_strides[1] = 64  # smaller than head_dim
    assert lib.heal_attn_decode_paged(ctypes.byref(a), None) == 3
    # the partials need a workspace: none, then too small -> HEAL_ERR_WORKSPACE before any launch
    assert lib.heal_attn_paged_workspace_bytes(ctypes.byref(_paged_args(heal))) > 0
    assert call() == 8
    assert call(workspace=FAKE, workspace_bytes=16) == 8
    assert call(batch=0) == 0


def test_gemm_quant_validation(heal):
    lib = heal.load()
    F16, BF16 = 2, 1
    args = lambda M=4, N=128, K=8, ah=FAKE, bh=FAKE, q=FAKE, s=FAKE, lda=8, ldb=8, ldq=128, lds=1, part=F16: (
        M, N, K, P(ah) if ah else None, None, None, lda, P(bh) if bh else None, None, None, ldb, part,
        P(q) if q else None, ldq, P(s) if s else None, lds, None)
    assert lib.heal_gemm_comp_quant_i16(*args(N=100, ldq=104)) == 2   # N not a multiple of 128
    assert lib.heal_gemm_comp_quant_i16(*args(M=-1)) == 2
    assert lib.heal_gemm_comp_quant_i16(*args(part=BF16)) == 5
    assert lib.heal_gemm_comp_quant_i16(*args(q=None)) == 1
    assert lib.heal_gemm_comp_quant_i16(*args(s=None)) == 1
    assert lib.heal_gemm_comp_quant_i16(*args(ah=None)) == 1
    assert lib.heal_gemm_comp_quant_i16(*args(ldq=64)) == 3
    assert lib.heal_gemm_comp_quant_i16(*args(N=256, ldq=256, lds=1)) == 3  # ld_s < N / 128
    assert lib.heal_gemm_comp_quant_i16(*args(q=MIS)) == 4
    assert lib.heal_gemm_comp_quant_i16(*args(ldq=132)) == 4
    assert lib.heal_gemm_comp_quant_i16(*args(s=FAKE + 2)) == 4
    assert lib.heal_gemm_comp_quant_i16(*args(M=0)) == 0


def test_channel_validation(heal):
    lib = heal.load()
    F32, BF16, F16, I16 = 0, 1, 2, 3
    ce = lambda x=FAKE, rows=4, cols=8, ld=8, T=8, out=FAKE: lib.heal_channel_exponents(
        P(x) if x else None, rows, cols, ld, T, P(out) if out else None, None)
    assert ce(rows=-1) == 2
    assert ce(T=200) == 2
    assert ce(out=None) == 1
    assert ce(x=None) == 1
    assert ce(ld=4) == 3
    assert ce(out=FAKE + 4) == 4
    assert ce(x=FAKE + 2) == 4
    assert ce(cols=0) == 0
    sp = lambda x=FAKE, xt=F32, rows=4, cols=8, ldx=8, part=F16, hi=FAKE, lo=FAKE, ldp=8, e=FAKE, c=FAKE, sign=1: (
        lib.heal_split_scaled(P(x) if x else None, xt, rows, cols, ldx, part, P(hi) if hi else None,
                              P(lo) if lo else None, ldp, P(e) if e else None, P(c) if c else None, sign, None))
    assert sp(sign=2) == 2
    assert sp(xt=I16) == 5
    assert sp(part=F32) == 5
    assert sp(c=None) == 1
    assert sp(hi=None) == 1
    assert sp(ldx=4) == 3
    assert sp(c=FAKE + 4) == 4
    assert sp(hi=MIS) == 4
    assert sp(ldp=12) == 4
    assert sp(rows=0) == 0
