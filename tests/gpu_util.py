"""Helpers for GPU tests: numpy <-> device tensors, tolerances, printing."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda"


def dev(a: np.ndarray) -> torch.Tensor:
    """uint16 (bf16 bits) -> bfloat16 tensor; float32 -> float32; int32 -> int32."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy float64 (bf16 widened exactly) or int32."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return (t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if t.dtype in (torch.int32, torch.int64):
        return t.numpy()
    return t.numpy().astype(np.float64)


def widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rms(a) -> float:
    return float(np.sqrt(np.mean(np.square(a))))


def say(*args):
    print("[gpu-test]", *args, flush=True)
    sys.stdout.flush()


def fp32_sum_bound(Xd: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """Bound on |fp32 sum - exact| for Y = X W^T summed in any order with
    fp32 products exact (bf16 inputs) or rounded (fp32 inputs):
    2 * K * 2^-24 * sum |x w|, per element."""
    K = Xd.shape[1]
    return 2.0 * K * 2.0 ** -24 * (np.abs(Xd) @ np.abs(Wd).T) + 1e-30
