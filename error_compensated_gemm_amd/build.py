"""Build libheal.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libheal.so")
SOURCES = ("split_quant.hip", "gemm_comp.hip", "attn.hip", "abi.hip")
# the decoder-block glue for the model-level check: a library of its own, outside HEAL's boundary
GLUE_LIB = os.path.join(HERE, "libheal_glue.so")
GLUE_SOURCES = ("glue.hip",)

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # IEEE fp32 division and square root: the INT16 quantiser's scale and codes depend on it
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # no packed-FP32 VALU instructions (the device pass honours this; the host pass warns that it does not know
    # the feature, which is harmless); packed_fp32_check() verifies the result
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep the gfx950 assembly of each source next to its object, for that check
    "-save-temps=obj",
]
PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def packed_fp32_check(obj: str) -> None:
    """Refuse a build whose gfx950 assembly holds a packed-FP32 VALU instruction."""
    asm = obj[:-2] + "-hip-amdgcn-amd-amdhsa-gfx950.s"
    if not os.path.exists(asm):
        raise RuntimeError(f"no device assembly for {os.path.basename(obj)} ({asm})")
    with open(asm) as f:
        hits = [l.strip() for l in f if PACKED_FP32.search(l)]
    if hits:
        raise RuntimeError(f"{os.path.basename(asm)}: {len(hits)} packed-FP32 instructions, e.g. {hits[0]}")


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
        if verbose and r.stderr.strip():
            print(r.stderr[-2000:])
        packed_fp32_check(obj)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + len(GLUE_SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES + GLUE_SOURCES))
    for lib, lib_objs in ((LIB, objs[:len(SOURCES)]), (GLUE_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *lib_objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed for {os.path.basename(lib)}:\n{r.stderr[-4000:]}")
        os.replace(tmp, lib)
    return LIB


ASAN_DIR = os.path.join(OBJ, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libheal_asan.so")


def asan_runtime() -> str | None:
    """The clang AddressSanitizer runtime that an -fsanitize=address host build links against, or None."""
    import glob

    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_asan() -> str:
    """libheal with its HOST code built under AddressSanitizer (the device code as usual), for running the
    argument validation of the C ABI under ASan on the CPU.  Rebuilt only when a source is newer."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    srcs = [os.path.join(CSRC, f) for f in SOURCES] + [os.path.join(CSRC, "heal_internal.h"),
                                                      os.path.join(HERE, "..", "include", "heal.h")]
    if os.path.exists(ASAN_LIB) and os.path.getmtime(ASAN_LIB) >= max(os.path.getmtime(f) for f in srcs):
        return ASAN_LIB
    flags = [f for f in HIPCC_FLAGS if f != "-save-temps=obj"] + ["-Xarch_host", "-fsanitize=address",
                                                                  "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src: str) -> str:
        obj = os.path.join(ASAN_DIR, src.replace(".hip", ".o"))
        r = subprocess.run([hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj], capture_output=True,
                           text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (asan) failed on {src}:\n{r.stderr[-4000:]}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-shared-libasan", *objs, "-o", ASAN_LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for the asan build:\n{r.stderr[-4000:]}")
    os.replace(ASAN_LIB + ".tmp", ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))
