#!/usr/bin/env python3
"""Benchmark of the HEAL hot path on one MI355X.

Headline (one JSON line on stdout): FP32-equivalent TFLOP/s of the error-compensated GEMM on the
Llama-3-8B projection shapes -- M in {1, 16, 2048} tokens x (K, N) in {(4096, 4096), (4096, 14336),
(14336, 4096)} -- with FP32 activations N(0, 1) carrying 1 % outlier channels x50 and bf16 weights N(0, 0.02)
(exact in FP16 after the per-row power-of-two prescale, so P = 2 products).  One step = for each of the
9 shapes: heal_split of the activations (FP32 -> FP16 hi + lo + row exponents) and heal_gemm_comp.  The
weights are split once at load time, outside the timed region.  Inputs are synthetic, seeded, resident in
HBM before timing starts.

Also reported in the same line:
  * "roofline" -- the dominant kernel of the step (the GEMM instantiation with the most time), its
    16-bit MFMA work per launch (P x 2MNK) over its average launch duration, measured with HIP events on
    the launch stream inside the timed region, against the 2516.6 TFLOP/s dense FP16 peak;
  * "cpu_baseline" -- the FP64 CPU oracle on a bounded row sample of the same 9 shapes (all host threads),
    and the GPU's error against it on those rows;
  * "rows" -- the other hot-path steps, timed after the headline loop: the activation split, the INT16
    quantiser, Dual-FP16 prefill (1 x 4096 x 32 heads x 128, causal), decode (64 x 8192 keys, GQA 32/8),
    the same decode over a paged cache (64-key pages, shuffled pool), the QKV projection with the INT16
    quantisation fused into the GEMM (against GEMM + quantiser) and the 8192^3 FP32 x FP32 GEMM (P = 3).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6  # MI355X dense FP16/BF16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-rows", action="store_true", help="skip the per-step measurements of the other rows")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="rows of each M=2048 shape in the CPU sample (2048: every output, about 10 s of FP64 work)")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (scale run for the HBM byte counters)")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="only print the HBM traffic summary of the rocprofv3 --pmc runs under DIR "
                         "(fetch/, write/, copy_fetch/, copy_write/)")
    ap.add_argument("--copy-mib", type=int, default=256, help="size of the calibration copy (MiB)")
    ap.add_argument("--only", choices=("prefill", "decode"),
                    help="only run 5 launches of that attention kernel on its workload (for counter runs)")
    ap.add_argument("--summarize-attn", metavar="DIR",
                    help="only print the counter summary of the attention runs under DIR (decode_fetch/, "
                         "decode_write/, copy_fetch/, copy_write/, prefill_sq/)")
    return ap.parse_args()


# ------------------------------------------------------------------ HBM traffic from stored counters
GEMM_SRC = os.path.join(ROOT, "error_compensated_gemm_amd", "csrc", "gemm_comp.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_comp_llama3_8b_hbm_traffic.md")
TRAFFIC_TAG = "traffic-json: "


def source_sha256(path):
    """SHA-256 of a C++ source with its comments and whitespace removed, so that the stored counters stay valid
    across comment edits and go stale with any change to the code itself."""
    import hashlib
    import re
    with open(path) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return hashlib.sha256("".join(src.split()).encode()).hexdigest()


def kernel_symbol(variant):
    """Template symbol of a GEMM variant name, as rocprofv3 prints it ("gemm_comp_kernel 256x128 P2" ->
    "gemm_comp_kernel<2, 256, 128, true, false, false, false, false>": FP16 parts, block tile, a_lo used, b_lo
    used, no fused quantisation, A given as parts, K not split)."""
    parts = variant.split()
    if len(parts) != 3 or parts[0] != "gemm_comp_kernel":
        return None
    bm, bn = parts[1].split("x")
    p = int(parts[2][1:])
    return f"gemm_comp_kernel<2, {bm}, {bn}, {str(p >= 2).lower()}, {str(p >= 3).lower()}, false, false, false>"


def stored_traffic(variant):
    """HBM bytes per launch of `variant` from the committed counter summary, or None when there is none or
    the GEMM source changed since the counters were taken."""
    sym = kernel_symbol(variant)
    if sym is None or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = next((json.loads(l[len(TRAFFIC_TAG):]) for l in f if l.startswith(TRAFFIC_TAG)), None)
    if rec is None or rec.get("source_sha256") != source_sha256(GEMM_SRC):
        return None
    k = rec.get("kernels", {}).get(sym)
    return None if k is None else k["traffic_bytes_per_launch"]


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy calibration: 5 copies of {mib} MiB done", flush=True)


def summarize_pmc(d, copy_mib):
    """Markdown summary of FETCH_SIZE / WRITE_SIZE (KiB per dispatch) for every GEMM kernel of a bench run,
    each scaled by the ratio of known bytes to the counter's reading for a plain copy of copy_mib MiB."""
    import csv
    import glob
    from collections import defaultdict

    def read(sub):
        vals = defaultdict(list)
        for f in glob.glob(os.path.join(d, sub, "*counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return vals

    fetch, write, cf, cw = read("fetch"), read("write"), read("copy_fetch"), read("copy_write")
    copy_name = lambda v: max((k for k in v if "copyBuffer" in k), key=lambda k: len(v[k]))
    nbytes = copy_mib * (1 << 20)
    cfk = sum(cf[copy_name(cf)]) / len(cf[copy_name(cf)])
    cwk = sum(cw[copy_name(cw)]) / len(cw[copy_name(cw)])
    ff, fw = nbytes / (cfk * 1024), nbytes / (cwk * 1024)
    kernels = {}
    rows = []
    for name in sorted(fetch):
        if "gemm_comp_kernel<" not in name and "gemm_skinny_kernel<" not in name:
            continue
        sym = name[name.index("gemm_"):].split(">")[0] + ">"
        fk = sum(fetch[name]) / len(fetch[name])
        wk = sum(write[name]) / len(write[name]) if name in write else float("nan")
        tb = fk * 1024 * ff + wk * 1024 * fw
        kernels[sym] = {"dispatches": len(fetch[name]), "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                        "traffic_bytes_per_launch": round(tb)}
        rows.append(f"| `{sym}` | {len(fetch[name])} | {fk:.1f} | {wk:.1f} | {tb / 1e6:.2f} |")
    rec = {"source_sha256": source_sha256(GEMM_SRC), "fetch_factor": round(ff, 4), "write_factor": round(fw, 4),
           "copy_mib": copy_mib, "kernels": kernels}
    print("# HBM traffic of the compensated-GEMM kernels: bench.py (Llama-3-8B linear shapes)\n")
    print("Commands (from the repository root on one MI355X, ROCm 7.2; D = an output directory):\n")
    print("```")
    print("cd /tmp && export TMPDIR=/tmp")
    for c, sub, prog in (("FETCH_SIZE", "fetch", "--steps 2 --warmup 1 --no-cpu --no-rows"),
                         ("WRITE_SIZE", "write", "--steps 2 --warmup 1 --no-cpu --no-rows"),
                         ("FETCH_SIZE", "copy_fetch", f"--copy-calibration {copy_mib}"),
                         ("WRITE_SIZE", "copy_write", f"--copy-calibration {copy_mib}")):
        print(f"timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d $D/{sub} -o pmc -- "
              f"python3 /root/repo/bench.py {prog}")
    print(f"python3 /root/repo/bench.py --summarize-pmc $D --copy-mib {copy_mib}")
    print("```\n")
    print(f"Scale: a plain device copy of {copy_mib} MiB reads {cfk:.0f} KiB by FETCH_SIZE and writes {cwk:.0f} KiB "
          f"by WRITE_SIZE per dispatch, so FETCH_SIZE x {ff:.3f} and WRITE_SIZE x {fw:.3f} give bytes.  The "
          "counters see traffic below the L2 (to the memory-side cache and HBM).\n")
    print("| kernel | dispatches | FETCH_SIZE (KiB/launch) | WRITE_SIZE (KiB/launch) | traffic (MB/launch) |")
    print("|---|---|---|---|---|")
    print("\n".join(rows))
    print("\nbench.py reads the record below and reports the traffic of its dominant kernel only while "
          "gemm_comp.hip still has this SHA-256.\n")
    print(TRAFFIC_TAG + json.dumps(rec))


def attn_decode_bytes(B=64, L=8192, Hq=32, Hkv=8, D=128):
    """algorithmic bytes of one decode call: K and V (INT16), their scales, q (INT16 + scale) and O (FP32)"""
    return 2.0 * B * L * Hkv * D * 2 + 2.0 * B * L * Hkv * 4 + B * Hq * D * (2 + 4)


def only_attention(heal, workloads, which):
    """5 launches of the a6 prefill (1 x 4096 x 32 x 128, causal) or the a7 decode (64 x 8192 keys, 32 / 8
    heads) on the bench's own inputs, nothing else: the program the attention counter runs profile."""
    import numpy as np
    import torch

    heal.load()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    if which == "prefill":
        Q, K, V = workloads.qkv_fp32(1, 4096, 32, 128, seed=2)
        (q, qs), (k, ks), (v, vs) = (heal.heal_qkv_quant_i16(dev(t[0])) for t in (Q, K, V))
        args = (q[None], qs[None], k[None], ks[None], v[None], vs[None])
        out = heal.heal_attn_dual_fp16(*args, causal=True)
        for _ in range(4):
            heal.heal_attn_dual_fp16(*args, causal=True, out=out)
    else:
        B, L, Hq, Hkv = 64, 8192, 32, 8
        k, ks = workloads.int16_cache_device(B, L, Hkv, 128, seed=3)
        v, vs = workloads.int16_cache_device(B, L, Hkv, 128, seed=4)
        q, qs = [dev(a) for a in workloads.int16_cache_host(B, 1, Hq, 128, seed=5)]
        out = torch.empty((B, 1, Hq, 128), dtype=torch.float32, device="cuda")
        ws = torch.empty(heal.heal_attn_workspace_bytes(heal.make_attn_args(q, qs, k, ks, v, vs, out, True)),
                         dtype=torch.uint8, device="cuda")
        for _ in range(5):
            heal.heal_attn_dual_fp16(q, qs, k, ks, v, vs, causal=True, out=out, workspace=ws)
    torch.cuda.synchronize()
    print(f"{which}: 5 launches done", flush=True)


def summarize_attn(d, copy_mib):
    """Markdown summary of the attention counter runs: decode HBM bytes (FETCH_SIZE / WRITE_SIZE scaled by a
    plain copy, as for the GEMM) and the prefill's matrix / vector occupancy (SQ counters, per SIMD)."""
    import csv
    import glob
    from collections import defaultdict

    def read(sub):
        vals = defaultdict(lambda: defaultdict(list))
        for f in glob.glob(os.path.join(d, sub, "*counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                vals[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
        return vals

    def trace(sub):
        durs = defaultdict(list)
        for f in glob.glob(os.path.join(d, sub, "*kernel_trace.csv")):
            for r in csv.DictReader(open(f)):
                durs[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
        return durs

    mean = lambda v: sum(v) / len(v)
    short = lambda n: n.replace("void ", "").replace("heal::(anonymous namespace)::", "").split("(")[0]
    cf, cw = read("copy_fetch"), read("copy_write")
    copy = lambda v: max((k for k in v if "copyBuffer" in k), key=lambda k: len(v[k]["FETCH_SIZE"] or
                                                                                 v[k]["WRITE_SIZE"]))
    nbytes = copy_mib * (1 << 20)
    ff = nbytes / (mean(cf[copy(cf)]["FETCH_SIZE"]) * 1024)
    fw = nbytes / (mean(cw[copy(cw)]["WRITE_SIZE"]) * 1024)
    fetch, write = read("decode_fetch"), read("decode_write")
    print("# Attention kernels: decode HBM traffic and prefill matrix / vector occupancy (bench.py workloads)\n")
    print("Commands (from the repository root on one MI355X, ROCm 7.2; D = an output directory):\n")
    print("```")
    print("cd /tmp && export TMPDIR=/tmp")
    for c, sub, prog in (("FETCH_SIZE", "decode_fetch", "--only decode"), ("WRITE_SIZE", "decode_write", "--only decode"),
                         ("FETCH_SIZE", "copy_fetch", f"--copy-calibration {copy_mib}"),
                         ("WRITE_SIZE", "copy_write", f"--copy-calibration {copy_mib}")):
        print(f"timeout -s KILL 60 rocprofv3 --pmc {c} --output-format csv -d $D/{sub} -o pmc -- "
              f"python3 /root/repo/bench.py {prog}")
    print(f"timeout -s KILL 60 rocprofv3 --pmc {' '.join(PREFILL_SQ)} --kernel-trace --output-format csv "
          "-d $D/prefill_sq -o pmc -- python3 /root/repo/bench.py --only prefill")
    print(f"python3 /root/repo/bench.py --summarize-attn $D --copy-mib {copy_mib}")
    print("```\n")
    algo = attn_decode_bytes()
    print(f"Decode (64 x 8192 keys, 32 query / 8 key-value heads): algorithmic {algo / 1e9:.3f} GB per call "
          f"(K and V INT16, their scales, q and O).  Counter scale from a plain {copy_mib} MiB copy: FETCH_SIZE x "
          f"{ff:.3f}, WRITE_SIZE x {fw:.3f}.\n")
    print("| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | bytes per launch | / algorithmic |")
    print("|---|---|---|---|---|---|")
    for name in sorted(fetch):
        if "attn_decode" not in name:
            continue
        fk = mean(fetch[name]["FETCH_SIZE"])
        wk = mean(write[name]["WRITE_SIZE"]) if name in write else float("nan")
        tb = fk * 1024 * ff + wk * 1024 * fw
        ratio = f"{tb / algo:.3f}" if "merge" not in name else "-"
        print(f"| `{short(name)}` | {len(fetch[name]['FETCH_SIZE'])} | {fk:.1f} | {wk:.1f} | {tb / 1e9:.4f} GB | "
              f"{ratio} |")
    sq, durs = read("prefill_sq"), trace("prefill_sq")
    print("\nPrefill (1 x 4096 x 32 x 128, causal, byte reading): counters summed over the chip, per launch; per-SIMD "
          "figures divide by 1024 SIMDs; the clock is GRBM_GUI_ACTIVE over 8 XCDs and the launch's duration under "
          "the counter run.\n")
    print("| kernel | launches | duration (us) | clock (GHz) | cycles / SIMD | MFMA busy / SIMD | VALU-MFMA "
          "co-issue / SIMD | VALU instructions (non-MFMA) / SIMD |")
    print("|---|---|---|---|---|---|---|---|")
    for name in sorted(sq):
        if "attn_prefill" not in name:
            continue
        c = {k: mean(v) for k, v in sq[name].items()}
        dur = mean(durs[name]) if durs.get(name) else float("nan")
        clk = c["GRBM_GUI_ACTIVE"] / 8 / dur / 1e9
        print(f"| `{short(name)}` | {len(sq[name]['GRBM_GUI_ACTIVE'])} | {dur * 1e6:.1f} | {clk:.2f} | "
              f"{dur * clk * 1e9:.3g} | {c['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024:.3g} | "
              f"{c['SQ_VALU_MFMA_COEXEC_CYCLES'] / 1024:.3g} | {(c['SQ_INSTS_VALU'] - c['SQ_INSTS_MFMA']) / 1024:.3g} |")
    print("\nSQ_VALU_MFMA_BUSY_CYCLES counts 32 cycles per v_mfma_f32_32x32x16_f16; a non-MFMA VALU instruction of "
          "a 64-wide wavefront takes 4 cycles on a 16-lane SIMD.")


PREFILL_SQ = ("GRBM_GUI_ACTIVE", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES",
              "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_BUSY_CYCLES")


class Timer:
    """HIP events on the current (launch) stream."""

    def __init__(self):
        import torch

        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, key, e0):
        e1 = self.torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.append((key, e0, e1))

    def durations(self):
        out = {}
        for key, a, b in self.pairs:
            out.setdefault(key, []).append(a.elapsed_time(b) * 1e-3)
        return out


def time_fn(fn, reps, warm=2):
    import torch

    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / reps


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.copy_mib)
        return
    if args.summarize_attn:
        summarize_attn(args.summarize_attn, args.copy_mib)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the hot path shards without communication and multi-GPU runs are not part of it",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import error_compensated_gemm_amd as heal
    import workloads

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.only:
        only_attention(heal, workloads, args.only)
        return
    heal.load()
    torch.cuda.set_device(0)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    # ---------------------------------------------------------------- set-up (untimed): weights split once
    shapes = [(M, K, N) for M in workloads.LLAMA3_8B_M for (K, N) in workloads.LLAMA3_8B_KN]
    weights = {}
    host_w = {}
    for (K, N) in workloads.LLAMA3_8B_KN:
        W = workloads.llama_weights_bf16(N, K, seed=1)
        host_w[(K, N)] = W
        wt = dev(W.view(np.int16)).view(torch.bfloat16)
        bh, _, eb = heal.heal_split(wt, residual=False)
        weights[(K, N)] = (bh, eb)
        del wt
    bufs = []
    host_x = {}
    for (M, K, N) in shapes:
        X = workloads.llama_activations(M, K, seed=1)
        host_x[(M, K)] = X
        x = dev(X)
        ah, al, ea = heal.heal_split(x)
        c = heal.heal_gemm_comp(ah, al, ea, *weights[(K, N)][:1], None, weights[(K, N)][1])
        bufs.append((M, K, N, x, ah, al, ea, c))
    torch.cuda.synchronize()
    # decode-sized M takes the entry point that splits A in the GEMM's prologue (the same bits as split +
    # GEMM, without the parts' round trip through HBM); prefill-sized M splits in its own pass
    # (one-row activations also leave the row exponent to the GEMM: a launch fewer, the same bits)
    fused = lambda M: M <= 64
    derived = lambda M: M == 1
    variants = {(M, K, N): heal.heal_gemm_comp_variant(M, N, K, 2) + (" FP32-A" if fused(M) else "")
                + (", exponent in the kernel" if derived(M) else "") for (M, K, N) in shapes}

    timer = Timer()

    def step(record):
        for (M, K, N, x, ah, al, ea, c) in bufs:
            bh, eb = weights[(K, N)]
            if derived(M):
                pass
            elif fused(M):
                heal.heal_row_exponents(x, exps=ea)
            else:
                heal.heal_split(x, hi=ah, lo=al, exps=ea)
            if record:
                e0 = timer.start()
            if fused(M):
                heal.heal_gemm_comp_f32a(x, None if derived(M) else ea, bh, None, eb, c=c)
            else:
                heal.heal_gemm_comp(ah, al, ea, bh, None, eb, c=c)
            if record:
                timer.stop((M, K, N), e0)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step(True)
    t1.record()
    torch.cuda.synchronize()
    total_s = t0.elapsed_time(t1) * 1e-3
    ms_per_step = total_s / args.steps * 1e3
    flops_step = sum(2.0 * M * N * K for (M, K, N) in shapes)
    value = flops_step / (total_s / args.steps) / 1e12

    durs = timer.durations()
    per_shape = {}
    by_variant = {}
    for (M, K, N) in shapes:
        d = durs[(M, K, N)]
        avg = sum(d) / len(d)
        per_shape[f"{M}x{K}x{N}"] = {
            "us": round(avg * 1e6, 2),
            "tflops_fp32eq": round(2.0 * M * N * K / avg / 1e12, 2),
            "hbm_gbs": round((2.0 * N * K + 8.0 * M * K + 4.0 * M * N) / avg / 1e9, 1),
            "kernel": variants[(M, K, N)],
        }
        v = by_variant.setdefault(variants[(M, K, N)], {"time": 0.0, "launches": 0, "mfma_flop": 0.0})
        v["time"] += sum(d)
        v["launches"] += len(d)
        v["mfma_flop"] += 2 * 2.0 * M * N * K * len(d)
    dom_name, dom = max(by_variant.items(), key=lambda kv: kv[1]["time"])
    avg_dur = dom["time"] / dom["launches"]
    achieved = dom["mfma_flop"] / dom["launches"] / avg_dur / 1e12
    roofline = {
        "bound": "mfma",
        "achieved": round(achieved, 1),
        "peak": PEAK_F16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_F16_TFLOPS, 4),
        "traffic": stored_traffic(dom_name),
        "kernel": dom_name,
        "avg_launch_us": round(avg_dur * 1e6, 2),
        "launches_per_step": dom["launches"] // args.steps,
        "work_per_launch": "P x 2MNK 16-bit MFMA flop (P = 2), averaged over the launches of this kernel",
    }

    result = {
        "metric": "FP32-equiv TFLOP/s of compensated GEMM + % of MFMA roofline; max rel err vs FP64",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "llama3_8b_linear: split(fp32 X) + compensated GEMM, P=2, 9 shapes (M <= 64: the split "
                        "in the GEMM's prologue; M = 1: the row exponent there too)",
            "shapes_MKN": [list(s) for s in shapes],
            "activations": "fp32 N(0,1), 1% channels x50",
            "weights": "bf16 N(0,0.02), pre-split to fp16 once",
            "flop_per_step_fp32eq": flops_step,
        },
        "roofline": roofline,
        "per_shape": per_shape,
    }

    # ------------------------------------------------------------------ CPU baseline: the FP64 oracle
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args, shapes, host_x, host_w, bufs, flops_step)

    if not args.no_rows:
        result["rows"] = other_rows(heal, workloads, dev)

    print(json.dumps(result), flush=True)


def cpu_baseline(args, shapes, host_x, host_w, bufs, flops_step):
    import ctypes

    import numpy as np

    import oracle

    lib = oracle.lib()
    try:
        threads = ctypes.CDLL("libgomp.so.1").omp_get_max_threads()
    except OSError:
        threads = os.cpu_count()
    wd = {}
    for (K, N), W in host_w.items():
        wd[(K, N)] = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    flops = 0.0
    t_cpu = 0.0
    errs, comps = [], []
    gpu_c = {(M, K, N): c for (M, K, N, x, ah, al, ea, c) in bufs}
    for (M, K, N) in shapes:
        rows = min(M, args.cpu_rows)
        X = host_x[(M, K)][:rows].astype(np.float64)
        t = time.perf_counter()
        C = oracle.gemm_f64(X, wd[(K, N)])
        t_cpu += time.perf_counter() - t
        flops += 2.0 * rows * K * N
        G = gpu_c[(M, K, N)][:rows].cpu().numpy().astype(np.float64)
        errs.append(float(np.linalg.norm(G - C) / np.linalg.norm(C)))
        absab = np.abs(X) @ np.abs(wd[(K, N)]).T
        comps.append(float(np.max(np.abs(G - C) / absab)))
    return {
        "value": round(flops / t_cpu / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"FP64 plain-C GEMM on the first min(M, {args.cpu_rows}) rows of each of the 9 shapes "
                  f"({flops:.3e} flop, {t_cpu:.1f} s)",
        "gpu_err_vs_fp64_on_sample": {"normwise_max": max(errs), "componentwise_max": max(comps)},
    }


def other_rows(heal, workloads, dev):
    """The remaining hot-path steps, each timed on its own workload with HIP events."""
    import numpy as np
    import torch

    rows = {}
    # a1: activation split, 2048 x 14336 fp32 -> fp16 hi + lo + exps (read 4 B, write 4 B per element)
    x = dev(workloads.llama_activations(2048, 14336, seed=1))
    hi, lo, e = heal.heal_split(x)
    t = time_fn(lambda: heal.heal_split(x, hi=hi, lo=lo, exps=e), 20)
    rows["a1_split_2048x14336"] = {"us": round(t * 1e6, 2), "gbs": round(x.numel() * 8 / t / 1e9, 1)}
    del x, hi, lo, e
    # a4 + a6: quantise Q, K, V [4096, 32, 128] then causal Dual-FP16 prefill
    Q, K, V = workloads.qkv_fp32(1, 4096, 32, 128, seed=2)
    qd, kd, vd = dev(Q[0]), dev(K[0]), dev(V[0])
    qkv = [heal.heal_qkv_quant_i16(t) for t in (qd, kd, vd)]
    def quant_all():
        for src, (q, s) in zip((qd, kd, vd), qkv):
            heal.heal_qkv_quant_i16(src, q=q, scale=s)
    t = time_fn(quant_all, 20)
    nel = 3 * qd.numel()
    rows["a4_quant_3x4096x32x128"] = {"us": round(t * 1e6, 2), "gbs": round(nel * (4 + 2 + 4 / 128) / t / 1e9, 1)}
    # the same values with each token's Q, K and V heads side by side ([4096, 96, 128], as a fused QKV
    # projection writes them): one launch, the same codes and scales
    fused = torch.cat([qd, kd, vd], dim=1)
    fq, fs = heal.heal_qkv_quant_i16(fused)
    t = time_fn(lambda: heal.heal_qkv_quant_i16(fused, q=fq, scale=fs), 20)
    rows["a4_quant_fused_qkv_4096x96x128"] = {"us": round(t * 1e6, 2),
                                              "gbs": round(nel * (4 + 2 + 4 / 128) / t / 1e9, 1)}
    del fused, fq, fs
    (q, qs), (k, ks), (v, vs) = qkv
    out = heal.heal_attn_dual_fp16(q[None], qs[None], k[None], ks[None], v[None], vs[None], causal=True)
    t = time_fn(lambda: heal.heal_attn_dual_fp16(q[None], qs[None], k[None], ks[None], v[None], vs[None],
                                                 causal=True, out=out), 10)
    fl = 4.0 * 128 * 32 * (4096 * 4097 / 2)
    rows["a6_prefill_1x4096x32x128_causal"] = {
        "us": round(t * 1e6, 2), "tflops_fp32eq": round(fl / t / 1e12, 2),
        "mfma_frac": round(8 * fl / 2 / t / 1e12 / PEAK_F16_TFLOPS, 4)}
    # the other readings of the Dual-FP16 pair: shift-10 (4 + 4 products), float-float (3 + 3 products)
    for reading, prods in (("shift10", 8), ("float", 6)):
        t = time_fn(lambda: heal.heal_attn_dual_fp16(q[None], qs[None], k[None], ks[None], v[None], vs[None],
                                                     causal=True, out=out, dual_split=reading), 10)
        rows[f"a6_prefill_1x4096x32x128_causal_{reading}"] = {
            "us": round(t * 1e6, 2), "tflops_fp32eq": round(fl / t / 1e12, 2),
            "mfma_frac": round(prods * fl / 2 / t / 1e12 / PEAK_F16_TFLOPS, 4)}
    del qd, kd, vd, qkv, q, k, v, out
    # a7: decode over an INT16 cache, 64 x 8192 keys, 32 q-heads / 8 kv-heads
    B, L, Hq, Hkv = 64, 8192, 32, 8
    k, ks = workloads.int16_cache_device(B, L, Hkv, 128, seed=3)
    v, vs = workloads.int16_cache_device(B, L, Hkv, 128, seed=4)
    q, qs = [dev(a) for a in workloads.int16_cache_host(B, 1, Hq, 128, seed=5)]
    out = torch.empty((B, 1, Hq, 128), dtype=torch.float32, device="cuda")
    args = heal.make_attn_args(q, qs, k, ks, v, vs, out, True)
    ws = torch.empty(heal.heal_attn_workspace_bytes(args), dtype=torch.uint8, device="cuda")
    t = time_fn(lambda: heal.heal_attn_dual_fp16(q, qs, k, ks, v, vs, causal=True, out=out, workspace=ws), 10)
    by = attn_decode_bytes(B, L, Hq, Hkv)
    rows["a7_decode_64x8192_gqa32_8"] = {"us": round(t * 1e6, 2), "gbs": round(by / t / 1e9, 1),
                                         "hbm_frac": round(by / t / 1e9 / PEAK_HBM_GBS, 4)}
    for reading in ("shift10", "float"):
        t = time_fn(lambda: heal.heal_attn_dual_fp16(q, qs, k, ks, v, vs, causal=True, out=out, workspace=ws,
                                                     dual_split=reading), 10)
        rows[f"a7_decode_64x8192_gqa32_8_{reading}"] = {"us": round(t * 1e6, 2), "gbs": round(by / t / 1e9, 1),
                                                        "hbm_frac": round(by / t / 1e9 / PEAK_HBM_GBS, 4)}
    # the same cache in 64-key pages of a shuffled pool (paged decode): pages gathered by index, no copy
    # of the keys on the timed path
    ps, npg = 64, L // 64
    g = torch.Generator(device="cpu")
    g.manual_seed(6)
    tab = torch.randperm(B * npg, generator=g).to(torch.int32).view(B, npg).to("cuda")
    def pool(t):
        p = torch.empty((B * npg, ps) + tuple(t.shape[2:]), dtype=t.dtype, device="cuda")
        p.index_copy_(0, tab.view(-1).long(), t.reshape((B * npg, ps) + tuple(t.shape[2:])))
        return p
    kp, ksp = pool(k), pool(ks)
    del k, ks
    vp, vsp = pool(v), pool(vs)
    del v, vs
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    q1, qs1, o1 = q[:, 0].contiguous(), qs[:, 0].contiguous(), out[:, 0].contiguous()
    pargs = heal.make_paged_args(q1, qs1, kp, ksp, vp, vsp, tab, lens, L, o1)
    pws = torch.empty(heal.heal_attn_paged_workspace_bytes(pargs), dtype=torch.uint8, device="cuda")
    t = time_fn(lambda: heal.heal_attn_decode_paged(q1, qs1, kp, ksp, vp, vsp, tab, lens, L, out=o1,
                                                    workspace=pws), 10)
    rows["a7p_paged_decode_64x8192_page64"] = {"us": round(t * 1e6, 2), "gbs": round(by / t / 1e9, 1),
                                               "hbm_frac": round(by / t / 1e9 / PEAK_HBM_GBS, 4)}
    # the same pool laid out head-major within each page ([P, Hkv, 64, D], passed through the strides): a
    # head's 64 keys are one contiguous 16 KB run
    def head_major(p):
        return p.transpose(1, 2).contiguous().transpose(1, 2)
    kp, ksp = head_major(kp), head_major(ksp)
    vp, vsp = head_major(vp), head_major(vsp)
    t = time_fn(lambda: heal.heal_attn_decode_paged(q1, qs1, kp, ksp, vp, vsp, tab, lens, L, out=o1,
                                                    workspace=pws), 10)
    rows["a7p_paged_decode_64x8192_page64_head_major"] = {"us": round(t * 1e6, 2), "gbs": round(by / t / 1e9, 1),
                                                          "hbm_frac": round(by / t / 1e9 / PEAK_HBM_GBS, 4)}
    del kp, ksp, vp, vsp, tab, lens, q, qs, out, ws, q1, qs1, o1, pws
    torch.cuda.empty_cache()
    # quantise-on-append: the Llama-3-8B QKV projection (2048 tokens x 4096 -> 6144 = 48 heads of 128, bf16
    # weights, P = 2) with the INT16 quantisation fused into the GEMM epilogue, against GEMM + quantiser
    X = dev(workloads.llama_activations(2048, 4096, seed=7))
    Wq = dev(workloads.llama_weights_bf16(6144, 4096, seed=7).view(np.int16)).view(torch.bfloat16)
    ah, al, ea = heal.heal_split(X)
    bh, _, eb = heal.heal_split(Wq, residual=False)
    qf, sf = heal.heal_gemm_comp_quant_i16(ah, al, ea, bh, None, eb)
    c = heal.heal_gemm_comp(ah, al, ea, bh, None, eb)
    qu, su = heal.heal_qkv_quant_i16(c.view(2048, 48, 128))
    def unfused():
        heal.heal_gemm_comp(ah, al, ea, bh, None, eb, c=c)
        heal.heal_qkv_quant_i16(c.view(2048, 48, 128), q=qu, scale=su)
    # the clock moves with heat and data, so the two are timed in turn, three times, best of each
    t_f = t_u = float("inf")
    for _ in range(3):
        t_f = min(t_f, time_fn(lambda: heal.heal_gemm_comp_quant_i16(ah, al, ea, bh, None, eb, q=qf, scale=sf), 10))
        t_u = min(t_u, time_fn(unfused, 10))
    fl = 2.0 * 2048 * 4096 * 6144
    rows["qkv_proj_quant_fused_2048x4096x6144"] = {
        "us": round(t_f * 1e6, 2), "unfused_us": round(t_u * 1e6, 2), "tflops_fp32eq": round(fl / t_f / 1e12, 1),
        "kernel": heal.heal_gemm_comp_variant(2048, 6144, 4096, 2)}
    del X, Wq, ah, al, ea, bh, eb, qf, sf, c, qu, su
    # split in the GEMM prologue: the three Llama-3-8B projections at M = 2048 and at M = 16, FP32
    # activations split inside the GEMM (row exponents + heal_gemm_comp_f32a) against the split pass + the
    # GEMM on its parts
    for M in (2048, 16):
        ops = []
        for K, N in ((4096, 4096), (4096, 14336), (14336, 4096)):
            X = dev(workloads.llama_activations(M, K, seed=8))
            W = dev(workloads.llama_weights_bf16(N, K, seed=8).view(np.int16)).view(torch.bfloat16)
            bh, _, eb = heal.heal_split(W, residual=False)
            ah, al, ea = heal.heal_split(X)
            c = heal.heal_gemm_comp(ah, al, ea, bh, None, eb)
            ops.append((X, bh, eb, ah, al, ea, c, heal.heal_row_exponents(X)))
        def split_then_gemm():
            for X, bh, eb, ah, al, ea, c, _ in ops:
                heal.heal_split(X, hi=ah, lo=al, exps=ea)
                heal.heal_gemm_comp(ah, al, ea, bh, None, eb, c=c)
        def split_in_prologue():
            for X, bh, eb, _, _, _, c, e2 in ops:
                heal.heal_row_exponents(X, exps=e2)
                heal.heal_gemm_comp_f32a(X, e2, bh, None, eb, c=c)
        t_f = t_u = float("inf")
        for _ in range(3):
            t_f = min(t_f, time_fn(split_in_prologue, 10))
            t_u = min(t_u, time_fn(split_then_gemm, 10))
        rows[f"split_in_prologue_{M}_llama3_8b_3_shapes"] = {"us": round(t_f * 1e6, 2),
                                                             "split_then_gemm_us": round(t_u * 1e6, 2)}
        del ops, X, W, bh, eb, ah, al, ea, c
    torch.cuda.empty_cache()
    # vendor library at equal matrix work: hipBLASLt (torch.matmul, FP16 in, FP32 accumulation inside) on
    # [M, 2K] x [2K, N] issues the same 16-bit MFMA work as the P = 2 compensated GEMM of each M = 2048 Llama
    # shape; timed in turn with ours, best of 3 (operands contiguous, no transposed views)
    t_ours = t_blas = 0.0
    pairs = {}
    for K, N in ((4096, 4096), (4096, 14336), (14336, 4096)):
        X = dev(workloads.llama_activations(2048, K, seed=9))
        W = dev(workloads.llama_weights_bf16(N, K, seed=9).view(np.int16)).view(torch.bfloat16)
        bh, _, eb = heal.heal_split(W, residual=False)
        ah, al, ea = heal.heal_split(X)
        c = heal.heal_gemm_comp(ah, al, ea, bh, None, eb)
        A2 = torch.randn((2048, 2 * K), device="cuda").to(torch.float16)
        B2 = torch.randn((2 * K, N), device="cuda").to(torch.float16)
        C2 = torch.matmul(A2, B2)
        b_best = o_best = float("inf")
        for _ in range(3):
            o_best = min(o_best, time_fn(lambda: heal.heal_gemm_comp(ah, al, ea, bh, None, eb, c=c), 10))
            b_best = min(b_best, time_fn(lambda: torch.matmul(A2, B2, out=C2), 10))
        t_ours += o_best
        t_blas += b_best
        pairs[f"2048x{K}x{N}"] = [round(o_best * 1e6, 1), round(b_best * 1e6, 1)]
        del X, W, bh, eb, ah, al, ea, c, A2, B2, C2
    rows["hipblaslt_fp16_equal_mfma_work_2048_llama3_8b_3_shapes"] = {
        "us": round(t_blas * 1e6, 2), "compensated_gemm_us": round(t_ours * 1e6, 2),
        "compensated_over_hipblaslt_time": round(t_ours / t_blas, 3), "per_shape_ours_hipblaslt_us": pairs}
    torch.cuda.empty_cache()
    # medium M (decode batches, short prefills): heal_gemm_comp_splitk, which cuts K across workgroups where the
    # plain launch leaves CUs idle, against heal_gemm_comp, on the three Llama projections; the weights rotate
    # through four copies so they stream from HBM, best of 3 in turn
    per = {}
    t_plain = t_split = 0.0
    for K, N in ((4096, 4096), (4096, 14336), (14336, 4096)):
        W = dev(workloads.llama_weights_bf16(N, K, seed=10).view(np.int16)).view(torch.bfloat16)
        bh, _, eb = heal.heal_split(W, residual=False)
        copies = [bh] + [bh.clone() for _ in range(3)]
        for M in (64, 128, 512):
            ah, al, ea = heal.heal_split(dev(workloads.llama_activations(M, K, seed=10)))
            c = heal.heal_gemm_comp(ah, al, ea, bh, None, eb)
            need = heal.heal_gemm_comp_workspace_bytes(M, N, K, 2)
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
            def rotate(fn):
                def run():
                    for b_ in copies:
                        fn(b_)
                return run
            plain = rotate(lambda b_: heal.heal_gemm_comp(ah, al, ea, b_, None, eb, c=c))
            split = rotate(lambda b_: heal.heal_gemm_comp_splitk(ah, al, ea, b_, None, eb, c=c, workspace=ws))
            p_best = s_best = float("inf")
            for _ in range(3):
                p_best = min(p_best, time_fn(plain, 5) / 4)
                s_best = min(s_best, time_fn(split, 5) / 4)
            t_plain += p_best
            t_split += s_best
            per[f"{M}x{K}x{N}"] = {"slices": heal.heal_gemm_comp_splitk_slices(M, N, K, 2),
                                   "splitk_us": round(s_best * 1e6, 1), "plain_us": round(p_best * 1e6, 1)}
        del W, bh, eb, copies, ah, al, ea, c, ws
    rows["gemm_splitk_medium_m_llama3_8b"] = {"us": round(t_split * 1e6, 1), "plain_us": round(t_plain * 1e6, 1),
                                              "per_shape": per}
    torch.cuda.empty_cache()
    # config 5a: 8192^3 FP32 x FP32, rows scaled by 10^U(-3,3), P = 3
    A, Bt = workloads.gemm_rowscaled(8192, 8192, 8192, seed=4)
    ah, al, ea = heal.heal_split(dev(A))
    bh, bl, eb = heal.heal_split(dev(Bt))
    c = heal.heal_gemm_comp(ah, al, ea, bh, bl, eb)
    t = time_fn(lambda: heal.heal_gemm_comp(ah, al, ea, bh, bl, eb, c=c), 5)
    fl = 2.0 * 8192 ** 3
    rows["gemm_8192cube_p3"] = {"us": round(t * 1e6, 1), "tflops_fp32eq": round(fl / t / 1e12, 1),
                                "mfma_frac": round(3 * fl / t / 1e12 / PEAK_F16_TFLOPS, 4),
                                "kernel": heal.heal_gemm_comp_variant(8192, 8192, 8192, 3)}
    return rows


if __name__ == "__main__":
    main()
