"""Model-level check of the HEAL path: a random-initialised Llama-style decoder stack run three ways,
  * HEAL: every projection is the compensated GEMM (FP32 activations, bf16 weights exact in FP16, P = 2;
    heal_split + heal_gemm_comp, or heal_gemm_comp_f32a for up to 64 rows, which gives the same bits), Q/K/V
    are INT16-quantised into the KV cache by heal_qkv_quant_i16 (one launch for all three), attention is
    heal_attn_dual_fp16 (prefill, then one decode step per token); the other block steps are the FP32 glue
    kernels of libheal_glue.so;
  * plain bf16: bf16 values between every op and in the KV cache, each op's arithmetic in FP32 on those values
    and its result rounded to bf16 (the kernel-boundary truncation the HEAL pages name as the source of
    irreproducibility);
  * FP64: ``oracle.stack``.
The FP64 model decodes greedily; the two 16-bit paths are then fed its tokens (teacher forcing) and their
argmax compared with its argmax at every step, and each also decodes on its own to find its first divergence.
Reported: per-step argmax agreement, first divergence, final-hidden normwise error against FP64, the median
time of one decode step (informational; the bf16 path is plain torch, not an inference engine), and the time per
output token of one decode step captured as a HIP graph for HEAL, a native bf16 pipeline and a global FP32
pipeline (TorchStep, plain torch with the HEAL path's fusion of the projections).

Run as a script for the full-size stack (32 layers, d 4096, 32/8 heads, FFN 14336, vocab 128256, 512-token
prompt, 64 steps; it needs ~100 GB of host memory for the FP64 weights):
    python tests/llama_stack.py --full
"""
from __future__ import annotations

import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import error_compensated_gemm_amd as heal  # noqa: E402
from oracle import stack as ostack  # noqa: E402

FULL = dict(layers=32, d=4096, hq=32, hkv=8, f=14336, vocab=128256, prompt=512, steps=64)
SMALL = dict(layers=2, d=1024, hq=8, hkv=2, f=3584, vocab=4096, prompt=64, steps=8)
EPS, THETA = 1e-5, 5e5


def glue():
    L = ctypes.CDLL(os.path.join(ROOT, "error_compensated_gemm_amd", "libheal_glue.so"))
    p, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    for name, args in (("glue_embed", [p, p, i64, i64, p, p]), ("glue_rmsnorm", [p, i64, i64, f32, p, p]),
                       ("glue_add_rmsnorm", [p, p, i64, i64, f32, p, p]),
                       ("glue_rope", [p, i64, i64, i64, i64, p, p]), ("glue_swiglu", [p, p, i64, p, p]),
                       ("glue_add", [p, p, i64, p]), ("glue_argmax", [p, i64, p, p])):
        getattr(L, name).argtypes = args
        getattr(L, name).restype = ctypes.c_int
    return L


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_weights(cfg: dict, seed: int) -> dict:
    """bf16 N(0, 0.02) weights on the device, drawn with torch's Philox generator from ``seed``."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    d, hq, hkv, f, V = cfg["d"], cfg["hq"], cfg["hkv"], cfg["f"], cfg["vocab"]

    def draw(r, c):
        return (torch.randn((r, c), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    w = {"emb": draw(V, d), "head": draw(V, d)}
    for l in range(cfg["layers"]):
        w[f"{l}.wq"], w[f"{l}.wk"], w[f"{l}.wv"] = draw(hq * 128, d), draw(hkv * 128, d), draw(hkv * 128, d)
        w[f"{l}.wo"] = draw(d, hq * 128)
        w[f"{l}.wg"], w[f"{l}.wu"], w[f"{l}.wd"] = draw(f, d), draw(f, d), draw(d, f)
    return w


def rope_table(positions: int) -> torch.Tensor:
    """cos and sin of pos * theta^(-i / 64), in FP64 rounded once to FP32, as [positions, 64, 2]."""
    i = np.arange(64, dtype=np.float64)
    ang = np.arange(positions, dtype=np.float64)[:, None] * np.power(THETA, -i / 64.0)[None, :]
    return torch.from_numpy(np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)).cuda()


class HealPath:
    def __init__(self, w: dict, cfg: dict, G):
        self.cfg, self.G = cfg, G
        d, hq, hkv = cfg["d"], cfg["hq"], cfg["hkv"]
        self.parts = {}
        for l in range(cfg["layers"]):
            self.parts[f"{l}.wqkv"] = heal.heal_split(torch.cat([w[f"{l}.wq"], w[f"{l}.wk"], w[f"{l}.wv"]]),
                                                      residual=False)[0::2]
            self.parts[f"{l}.wgu"] = heal.heal_split(torch.cat([w[f"{l}.wg"], w[f"{l}.wu"]]), residual=False)[0::2]
            for n in ("wo", "wd"):
                self.parts[f"{l}.{n}"] = heal.heal_split(w[f"{l}.{n}"], residual=False)[0::2]
        self.parts["head"] = heal.heal_split(w["head"], residual=False)[0::2]
        self.emb = w["emb"]
        Lmax = cfg["prompt"] + cfg["steps"]
        self.cs = rope_table(Lmax)
        # per layer, the INT16 Q, K and V heads of every position side by side ([Lmax, hq + 2 hkv, 128]) and
        # their scales, so that one quantiser launch fills all three; attention reads K and V as strided views
        H = hq + 2 * hkv
        self.qkv = [torch.zeros((Lmax, H, 128), dtype=torch.int16, device="cuda") for _ in range(cfg["layers"])]
        self.qkvs = [torch.zeros((Lmax, H), dtype=torch.float32, device="cuda") for _ in range(cfg["layers"])]

    def linear(self, x, name, rows=slice(None)):
        """x W^T for the FP16 parts of ``name`` (``rows`` selects a block of W's rows).  Up to 64 rows of x are
        split inside the GEMM's prologue (the same bits as heal_split + heal_gemm_comp, one launch fewer), and one
        row also has its exponent derived there."""
        bh, eb = self.parts[name]
        bh, eb = bh[rows], eb[rows]
        if x.shape[0] == 1:  # the GEMM derives the row exponent itself: one launch
            return heal.heal_gemm_comp_f32a(x, None, bh, None, eb)
        if x.shape[0] <= 64:
            return heal.heal_gemm_comp_f32a(x, heal.heal_row_exponents(x), bh, None, eb)
        ah, al, ea = heal.heal_split(x)
        return heal.heal_gemm_comp(ah, al, ea, bh, None, eb)

    def add_norm(self, x, r):
        """x += r, then rmsnorm(x), in one launch"""
        y = torch.empty_like(x)
        assert self.G.glue_add_rmsnorm(_p(x), _p(r), x.shape[0], x.shape[1], EPS, _p(y), _s()) == 0
        return y

    def norm(self, x):
        y = torch.empty_like(x)
        assert self.G.glue_rmsnorm(_p(x), x.shape[0], x.shape[1], EPS, _p(y), _s()) == 0
        return y

    def forward(self, ids: np.ndarray, pos0: int):
        return self.forward_dev(torch.from_numpy(np.asarray(ids, np.int32)).cuda(), pos0)

    def forward_dev(self, idt: torch.Tensor, pos0: int):
        """forward() on token ids already in device memory (so that a decode step can be captured)"""
        cfg, G = self.cfg, self.G
        T, d, hq, hkv = idt.numel(), cfg["d"], cfg["hq"], cfg["hkv"]
        x = torch.empty((T, d), dtype=torch.float32, device="cuda")
        assert G.glue_embed(_p(self.emb), _p(idt), T, d, _p(x), _s()) == 0
        H, F = hq + 2 * hkv, cfg["f"]
        h = self.norm(x)
        for l in range(cfg["layers"]):
            qkv = self.linear(h, f"{l}.wqkv")  # [T, (hq + 2 hkv) 128]
            assert G.glue_rope(_p(qkv), T, hq + hkv, qkv.stride(0), pos0, _p(self.cs), _s()) == 0  # Q and K heads
            c, cs = self.qkv[l], self.qkvs[l]
            heal.heal_qkv_quant_i16(qkv.view(T, H, 128), q=c[pos0:pos0 + T], scale=cs[pos0:pos0 + T])
            n = pos0 + T
            kh, vh = slice(hq, hq + hkv), slice(hq + hkv, H)
            a = heal.heal_attn_dual_fp16(c[None, pos0:n, :hq], cs[None, pos0:n, :hq], c[None, :n, kh],
                                         cs[None, :n, kh], c[None, :n, vh], cs[None, :n, vh], causal=True)
            o = self.linear(a.view(T, hq * 128), f"{l}.wo")
            h = self.add_norm(x, o)  # the residual add and the FFN's norm
            if T == 1:  # gate and up in one GEMM: the two halves of its one output row are each contiguous
                gu = self.linear(h, f"{l}.wgu")
                gte, up = gu[:, :F], gu[:, F:]
            else:
                gte, up = self.linear(h, f"{l}.wgu", slice(0, F)), self.linear(h, f"{l}.wgu", slice(F, 2 * F))
            act = torch.empty((T, F), dtype=torch.float32, device="cuda")
            assert G.glue_swiglu(_p(gte), _p(up), T * F, _p(act), _s()) == 0
            dn = self.linear(act, f"{l}.wd")
            if l + 1 < cfg["layers"]:
                h = self.add_norm(x, dn)  # the residual add and the next layer's attention norm
            else:
                assert G.glue_add(_p(x), _p(dn), x.numel(), _s()) == 0
        hn = self.norm(x[-1:].contiguous())
        logits = self.linear(hn, "head")
        am = torch.empty((1,), dtype=torch.int32, device="cuda")
        assert G.glue_argmax(_p(logits), logits.numel(), _p(am), _s()) == 0
        return hn[0], logits[0], am


class Bf16Path:
    """bf16 values between ops and in the cache; each op computes in FP32 on them and rounds its result."""

    def __init__(self, w: dict, cfg: dict):
        self.cfg = cfg
        self.wt = {k: v.float().t().contiguous() for k, v in w.items() if k not in ("emb",)}
        self.emb = w["emb"]
        Lmax = cfg["prompt"] + cfg["steps"]
        ang = torch.from_numpy(np.arange(Lmax, dtype=np.float64)[:, None]
                               * np.power(THETA, -np.arange(64, dtype=np.float64) / 64.0)[None, :])
        self.cos, self.sin = ang.cos().float().cuda(), ang.sin().float().cuda()
        self.k = [None] * cfg["layers"]
        self.v = [None] * cfg["layers"]

    @staticmethod
    def r(x):
        return x.to(torch.bfloat16).float()

    def norm(self, x):
        return self.r(x * torch.rsqrt((x * x).mean(-1, keepdim=True) + EPS))

    def rope(self, x, pos0):  # x [T, H, 128]
        T = x.shape[0]
        c, s = self.cos[pos0:pos0 + T, None, :], self.sin[pos0:pos0 + T, None, :]
        a, b = x[..., :64], x[..., 64:]
        return self.r(torch.cat([a * c - b * s, b * c + a * s], -1))

    def forward(self, ids: np.ndarray, pos0: int):
        cfg = self.cfg
        T, hq, hkv = len(ids), cfg["hq"], cfg["hkv"]
        g = hq // hkv
        x = self.emb[torch.from_numpy(np.asarray(ids, np.int64)).cuda()].float()
        for l in range(cfg["layers"]):
            h = self.norm(x)
            q = self.rope(self.r(h @ self.wt[f"{l}.wq"]).view(T, hq, 128), pos0)
            k = self.rope(self.r(h @ self.wt[f"{l}.wk"]).view(T, hkv, 128), pos0)
            v = self.r(h @ self.wt[f"{l}.wv"]).view(T, hkv, 128)
            self.k[l] = k if pos0 == 0 else torch.cat([self.k[l], k])
            self.v[l] = v if pos0 == 0 else torch.cat([self.v[l], v])
            K, V = self.k[l], self.v[l]
            L = K.shape[0]
            qh = q.view(T, hkv, g, 128).permute(1, 2, 0, 3).contiguous()          # [hkv, g, T, 128]
            s = torch.matmul(qh, K.permute(1, 2, 0).contiguous()[:, None]) / np.sqrt(128.0)  # [hkv, g, T, L]
            mask = torch.arange(L, device="cuda")[None, :] > (pos0 + torch.arange(T, device="cuda"))[:, None]
            s = s.masked_fill(mask, float("-inf"))
            p = torch.softmax(s, -1)
            o = torch.matmul(self.r(p), V.permute(1, 0, 2).contiguous()[:, None])  # [hkv, g, T, 128]
            a = self.r(o.permute(2, 0, 1, 3).reshape(T, hq * 128))
            x = self.r(x + self.r(a @ self.wt[f"{l}.wo"]))
            h = self.norm(x)
            gte, up = self.r(h @ self.wt[f"{l}.wg"]), self.r(h @ self.wt[f"{l}.wu"])
            act = self.r(gte / (1.0 + torch.exp(-gte)) * up)
            x = self.r(x + self.r(act @ self.wt[f"{l}.wd"]))
        hn = self.norm(x[-1:])
        logits = (hn @ self.wt["head"])[0]
        return hn[0], logits, torch.argmax(logits)


class TorchStep:
    """One decode step of the same stack in plain torch in one dtype, for the time-per-token comparison:
    bfloat16 is the native 16-bit pipeline (bf16 weights, activations and KV cache; matrix products on the
    16-bit matrix units), float32 the global FP32 pipeline (FP32 weights, activations and KV cache; TF32 off).
    The projections are fused as the HEAL path fuses them (Q, K and V in one product, gate and up in one), the
    cache holds ``ctx`` positions, and attention at position ``pos`` is two batched products over the first
    pos + 1 keys around an FP32 softmax; norms also reduce in FP32.  It times the launch structure; its
    arithmetic is not checked against FP64."""

    def __init__(self, w: dict, cfg: dict, dtype, ctx: int):
        self.cfg, self.dt = cfg, dtype
        L = cfg["layers"]
        t = lambda *ks: torch.cat([w[k] for k in ks]).to(dtype)  # [N, K], as torch.nn.Linear holds it
        self.wqkv = [t(f"{l}.wq", f"{l}.wk", f"{l}.wv") for l in range(L)]
        self.wo = [t(f"{l}.wo") for l in range(L)]
        self.wgu = [t(f"{l}.wg", f"{l}.wu") for l in range(L)]
        self.wd = [t(f"{l}.wd") for l in range(L)]
        self.head = t("head")
        self.emb = w["emb"].to(dtype)
        cs = rope_table(ctx)
        self.cos, self.sin = cs[..., 0].to(dtype), cs[..., 1].to(dtype)
        self.k = [torch.zeros((cfg["hkv"], ctx, 128), dtype=dtype, device="cuda") for _ in range(L)]
        self.v = [torch.zeros((cfg["hkv"], ctx, 128), dtype=dtype, device="cuda") for _ in range(L)]

    def rms(self, x):
        xf = x.float()
        return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + EPS)).to(self.dt)

    def rope(self, x, pos):  # x [H, 128]
        a, b = x[:, :64], x[:, 64:]
        c, s = self.cos[pos], self.sin[pos]
        return torch.cat([a * c - b * s, b * c + a * s], -1)

    def step(self, ids: torch.Tensor, pos: int):
        cfg = self.cfg
        hq, hkv, F = cfg["hq"], cfg["hkv"], cfg["f"]
        g = hq // hkv
        lin = torch.nn.functional.linear  # x W^T
        x = self.emb[ids.long()]  # [1, d]
        for l in range(cfg["layers"]):
            qkv = lin(self.rms(x), self.wqkv[l])
            q = self.rope(qkv[0, :hq * 128].view(hq, 128), pos)
            k = self.rope(qkv[0, hq * 128:(hq + hkv) * 128].view(hkv, 128), pos)
            self.k[l][:, pos] = k
            self.v[l][:, pos] = qkv[0, (hq + hkv) * 128:].view(hkv, 128)
            K, V = self.k[l][:, :pos + 1], self.v[l][:, :pos + 1]  # [hkv, pos + 1, 128], rows contiguous
            qt = q.view(hkv, g, 128).transpose(1, 2).contiguous()  # [hkv, 128, g]
            sc = torch.matmul(K, qt).float() * (1.0 / np.sqrt(128.0))  # [hkv, pos + 1, g]
            pt = torch.softmax(sc, dim=1).to(self.dt).transpose(1, 2).contiguous()  # [hkv, g, pos + 1]
            o = torch.matmul(pt, V)  # [hkv, g, 128]
            x = x + lin(o.reshape(1, hq * 128), self.wo[l])
            gu = lin(self.rms(x), self.wgu[l])
            x = x + lin(torch.nn.functional.silu(gu[:, :F]) * gu[:, F:], self.wd[l])
        return torch.argmax(lin(self.rms(x), self.head))


def graph_ms(fn, reps: int = 20) -> float:
    """GPU time of ``fn()`` (one decode step), captured once as a HIP graph and replayed (each replay rewrites the
    same cache slot with the same values)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def graph_step_ms(path: HealPath, tok: int, pos: int, reps: int = 20) -> float:
    """GPU time of one decode step of the HEAL path, captured once as a HIP graph and replayed."""
    ids = torch.tensor([tok], dtype=torch.int32, device="cuda")
    return graph_ms(lambda: path.forward_dev(ids, pos), reps)


def tpot_compare(w: dict, cfg: dict, tok: int, pos: int, heal_ms: float) -> dict:
    """Time per output token of one decode step at position ``pos``, each pipeline captured as a HIP graph and
    replayed: HEAL (measured by the caller), native bf16 and global FP32 (TorchStep); the ratios the pages report
    are FP32 / bf16 (the global FP32 pipeline's overhead) and HEAL / bf16."""
    torch.backends.cuda.matmul.allow_tf32 = False
    torch.set_float32_matmul_precision("highest")
    out = {"position": pos, "heal_ms": heal_ms}
    ids = torch.tensor([tok], dtype=torch.int32, device="cuda")
    for name, dt in (("bf16", torch.bfloat16), ("fp32", torch.float32)):
        st = TorchStep(w, cfg, dt, pos + 1)
        out[f"{name}_ms"] = graph_ms(lambda: st.step(ids, pos))
        del st
        torch.cuda.empty_cache()
    out["fp32_over_bf16"] = out["fp32_ms"] / out["bf16_ms"]
    out["heal_over_bf16"] = heal_ms / out["bf16_ms"]
    out["heal_over_fp32"] = heal_ms / out["fp32_ms"]
    return out


def _nw(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def run(cfg: dict, seed: int = 0, log=print) -> dict:
    t0 = time.time()
    w = make_weights(cfg, seed)
    host = {k: v.view(torch.int16).cpu().numpy().view(np.uint16) for k, v in w.items()}
    prompt = np.random.default_rng(seed).integers(0, cfg["vocab"], cfg["prompt"])
    log(f"[stack] weights ready ({time.time() - t0:.0f} s)")
    ref = ostack.Stack(host, cfg["layers"], cfg["hq"], cfg["hkv"], EPS, THETA, cfg["prompt"] + cfg["steps"])
    del host  # the FP64 model holds the only host copy of the bf16 weights, and drops each once widened
    t_ref = time.time()
    hid, lg = ref.forward(prompt, 0)
    toks, hids, gaps = [], [], []
    for s in range(cfg["steps"]):
        if s:
            hid, lg = ref.forward([toks[-1]], cfg["prompt"] + s - 1)
        top2 = np.sort(lg)[-2:]
        toks.append(int(np.argmax(lg)))
        hids.append(hid)
        gaps.append(float(top2[1] - top2[0]))
        log(f"[stack] fp64 step {s}: token {toks[-1]} (top-2 gap {gaps[-1]:.3e}, {time.time() - t0:.0f} s)")
    t_ref = time.time() - t_ref
    del ref
    G = glue()
    out = {"config": cfg, "seed": seed, "fp64_tokens": toks, "fp64_top2_gap_min": min(gaps),
           "fp64_forward_s": round(t_ref, 2)}
    for name, make in (("heal", lambda: HealPath(w, cfg, G)), ("bf16", lambda: Bf16Path(w, cfg))):
        path = make()
        agree, errs, step_ms = [], [], []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for mode in ("teacher_forced", "free"):
            h, logits, am = path.forward(prompt, 0)
            tok = int(am.item())
            first_div = None
            for s in range(cfg["steps"]):
                if s:
                    feed = toks[s - 1] if mode == "teacher_forced" else tok
                    e0.record()
                    h, logits, am = path.forward([feed], cfg["prompt"] + s - 1)
                    e1.record()
                    tok = int(am.item())
                    step_ms.append(e0.elapsed_time(e1))
                if mode == "teacher_forced":
                    agree.append(tok == toks[s])
                    errs.append(_nw(h.double().cpu().numpy(), hids[s]))
                elif first_div is None and tok != toks[s]:
                    first_div = s
            if mode == "free":
                out[name] = {"teacher_forced_agreement": sum(agree) / len(agree),
                             "disagreeing_steps": [s for s, a in enumerate(agree) if not a],
                             "free_running_first_divergence": first_div,
                             "final_hidden_normwise_err_max": max(errs),
                             "final_hidden_normwise_err_mean": float(np.mean(errs)),
                             "decode_step_ms_median": float(np.median(step_ms))}
                if name == "heal":
                    out[name]["decode_step_ms_hip_graph"] = graph_step_ms(path, toks[-1], cfg["prompt"] + cfg["steps"] - 1)
        log(f"[stack] {name}: {json.dumps(out[name])} ({time.time() - t0:.0f} s)")
        del path
        torch.cuda.empty_cache()
    pos = cfg["prompt"] + cfg["steps"] - 1
    out["tpot"] = tpot_compare(w, cfg, toks[-1], pos, out["heal"]["decode_step_ms_hip_graph"])
    log(f"[stack] tpot: {json.dumps(out['tpot'])} ({time.time() - t0:.0f} s)")
    return out


def summarize_trace(d: str, steps: int = 20) -> None:
    """Markdown breakdown of the replayed HEAL decode steps in a rocprofv3 kernel trace of this script.  Every
    HEAL forward ends with the glue argmax kernel and the graph replays are the last HEAL forwards, so the last
    ``steps`` argmax-terminated runs of dispatches are the timed replays."""
    import csv
    import glob
    from collections import defaultdict

    short = lambda n: n.replace("void ", "").replace("(anonymous namespace)::", "").replace("heal::", "").split("(")[0]
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short(r["Kernel_Name"])))
    rows.sort()
    ends = [i for i, r in enumerate(rows) if r[2] == "argmax_kernel"]
    assert len(ends) > steps, f"{len(ends)} HEAL forwards in the trace"
    per = defaultdict(lambda: [0, 0])  # name -> [launches, ns] over the replays
    wall = busy = launches = 0
    for k in range(len(ends) - steps, len(ends)):
        seg = rows[ends[k - 1] + 1:ends[k] + 1]
        wall += seg[-1][1] - seg[0][0]
        for t0, t1, n in seg:
            busy += t1 - t0
            per[n][0] += 1
            per[n][1] += t1 - t0
        launches += len(seg)
    print("# Decode step of the HEAL decoder stack (32 layers, d 4096, 32/8 heads, FFN 14336, vocabulary 128256), "
          "replayed as a HIP graph: per-kernel time\n")
    print("Command (from the repository root on one MI355X, ROCm 7.2; D = an output directory):\n")
    print("```")
    print("cd /tmp && export TMPDIR=/tmp")
    print("rocprofv3 --kernel-trace --output-format csv -d $D -o run -- python3 /root/repo/tests/llama_stack.py --full")
    print("python3 /root/repo/tests/llama_stack.py --summarize-trace $D")
    print("```\n")
    print(f"Over the last {steps} replays (context 575 tokens), per step: {launches / steps:.0f} kernel launches, "
          f"{wall / steps / 1e3:.1f} us from the first kernel's start to the last one's end, of which "
          f"{busy / steps / 1e3:.1f} us inside kernels and {(wall - busy) / steps / 1e3:.1f} us between them "
          f"({(wall - busy) / launches / 1e3:.2f} us per launch).  Timestamps are the tracer's; the untraced "
          "replay time is printed by the script itself.\n")
    print("| kernel | launches per step | us per launch | us per step | share of kernel time |")
    print("|---|---|---|---|---|")
    for n, (c, ns) in sorted(per.items(), key=lambda kv: -kv[1][1]):
        print(f"| `{n}` | {c / steps:.0f} | {ns / c / 1e3:.2f} | {ns / steps / 1e3:.1f} | {ns / busy:.1%} |")


if __name__ == "__main__":
    if "--summarize-trace" in sys.argv:
        summarize_trace(sys.argv[sys.argv.index("--summarize-trace") + 1])
        sys.exit(0)
    cfg = FULL if "--full" in sys.argv else SMALL
    res = run(cfg, log=lambda m: print(m, flush=True))
    print(json.dumps(res), flush=True)
