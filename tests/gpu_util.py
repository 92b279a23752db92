"""Helpers shared by the GPU parity tests (host <-> device copies and error measures)."""
import numpy as np
import torch


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    """16-bit patterns of an int16 / float16 / bfloat16 tensor as uint16"""
    return host(t.view(torch.int16)).view(np.uint16)


def normwise(x: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((np.asarray(x, np.float64) - ref).ravel()) / (den if den > 0 else 1.0))


def banner(msg: str):
    print(f"[gpu-case] {msg}", flush=True)


def worst_row(x: np.ndarray, ref: np.ndarray) -> float:
    """Largest normwise relative error of one output row (the last axis: one (b, i, h) row of an attention
    output); a row whose reference is all zero counts its largest absolute value."""
    d = ref.shape[-1]
    x = np.asarray(x, np.float64).reshape(-1, d)
    ref = np.asarray(ref, np.float64).reshape(-1, d)
    num = np.linalg.norm(x - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    err = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.abs(x).max(axis=1))
    return float(err.max()) if err.size else 0.0


def attn_row_errors(got, q, qs, k, ks, v, vs, causal, ref, rows=None):
    """Per-row errors of an attention output against the FP64 oracle on the dequantised inputs:
    (the largest normwise relative error of one (b, i, h) row, the largest row error measured against
    sum_j p_j |v_j|, the row's output with every value replaced by its magnitude).  The second is the row's
    error free of cancellation in the weighted sum, the natural per-row scale of an FP32 accumulation of
    p_j v_j."""
    import oracle

    qd, kd, vd = oracle.dequant_i16(q, qs), oracle.dequant_i16(k, ks), oracle.dequant_i16(v, vs)
    ref_abs = oracle.attn_f64(qd, kd, np.abs(vd), causal, rows=rows)
    d = ref.shape[-1]
    g = np.asarray(got, np.float64).reshape(-1, d)
    r = np.asarray(ref, np.float64).reshape(-1, d)
    den = np.linalg.norm(np.asarray(ref_abs, np.float64).reshape(-1, d), axis=1)
    num = np.linalg.norm(g - r, axis=1)
    cond = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.abs(g).max(axis=1))
    return worst_row(got, ref), float(cond.max()) if cond.size else 0.0
