"""Build libheal.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures
import os
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
    # no packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


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


if __name__ == "__main__":
    print(build(verbose=True))
