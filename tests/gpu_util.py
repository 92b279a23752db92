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
