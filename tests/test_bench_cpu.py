"""Host-side checks of bench.py's bookkeeping: the kernel-to-source table its counter summaries rely on, and the
stored traffic records in profiles/."""
import json
import os
import re

import bench

LIB_SOURCES = ("split_quant.hip", "gemm_comp.hip", "attn.hip", "abi.hip")


def _kernels(src):
    """Names of the __global__ functions a source defines."""
    text = open(os.path.join(bench.CSRC, src)).read()
    names = set()
    for m in re.finditer(r"__global__", text):
        hit = re.search(r"\bvoid\s+([A-Za-z_][A-Za-z_0-9]*)\s*\(", text[m.end():m.end() + 400])  # kernels return void
        if hit:
            names.add(hit.group(1))
    return names


def test_every_kernel_maps_to_its_source():
    # a kernel the table misses (or maps to another file) drops out of the FETCH_SIZE / WRITE_SIZE summaries
    seen = 0
    for src in LIB_SOURCES:
        for name in _kernels(src):
            assert bench.kernel_source(name + "<") == src or bench.kernel_source(name) == src, (name, src)
            seen += 1
    assert seen >= 14


def test_prefixes_do_not_shadow_each_other():
    # "gemm_stream_kernel" must not claim "gemm_stream_sk_kernel" (or the other way round)
    assert bench.kernel_source("gemm_stream_sk_kernel<2, 4, true, false, 1>") == "gemm_comp.hip"
    assert bench.kernel_source("gemm_stream_kernel<2, 4, 4, 3840, true, false, 2>") == "gemm_comp.hip"
    assert bench.kernel_source("not_a_heal_kernel") is None


def test_stored_traffic_records_parse():
    # every traffic record names a known source and a positive byte count per launch
    n = 0
    for f in sorted(os.listdir(bench.PROFILES)):
        if not f.endswith("_hbm_traffic.md"):
            continue
        lines = [l for l in open(os.path.join(bench.PROFILES, f)) if l.startswith(bench.TRAFFIC_TAG)]
        assert len(lines) == 1, f
        rec = json.loads(lines[0][len(bench.TRAFFIC_TAG):])
        assert rec["fetch_factor"] > 0 and rec["write_factor"] > 0
        for sym, k in rec["kernels"].items():
            assert k["source"] == bench.kernel_source(sym), (f, sym)
            assert k["traffic_bytes_per_launch"] > 0 and k["dispatches"] > 0
            assert re.fullmatch(r"[0-9a-f]{64}", k["source_sha256"])
            n += 1
    assert n > 0
