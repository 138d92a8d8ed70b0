"""Helpers for GPU tests: numpy <-> device tensors, tolerances, printing."""
from __future__ import annotations

import sys

import numpy as np
import torch

from moe_block_skinny_amd import synth

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


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Exact values rounded as the GPU rounds its fp32 output: to fp32, then
    to bf16 (nearest, ties to even); returned widened to float64."""
    b = synth.to_bf16_bits(np.asarray(a, np.float64).astype(np.float32))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# Block output bars (bf16 output, fp32 internals).
STATED_BAR = 2e-2     # max|err| <= 2e-2 * rms(ref), the stated bar
FP32_BLOCK = 1e-3     # bound on the fp32-internal error of a block output, x rms(ref)


def check_block_output(g: np.ndarray, ref: np.ndarray) -> tuple:
    """Assert the bf16 block-output bars; return (max|err|/rms, the same for
    the exact result rounded to bf16).

    Per element: |g - ref| <= |bf16(ref) - ref| + 2 * FP32_BLOCK * rms.  The
    GPU rounds its fp32 result r = ref + delta (|delta| <= FP32_BLOCK * rms)
    to bf16; if that rounds like ref does, the error is ref's own rounding
    error; if not, a rounding midpoint lies between ref and r, so ref's own
    rounding error is at least half an ulp minus |delta| and the GPU's at
    most half an ulp plus |delta|.
    The stated bar max|err| <= 2e-2 rms is asserted wherever the exact result
    rounded to bf16 leaves room for it (its own max error plus 2 * FP32_BLOCK
    below the bar); outputs reaching ~6 rms can exceed it by rounding alone.
    """
    scale = rms(ref)
    err = np.abs(g - ref)
    rnd = np.abs(bf16_round(ref) - ref)
    bad = err > rnd + 2 * FP32_BLOCK * scale
    assert not bad.any(), "bf16-aware per-element bar: %d elements, worst excess %.3g rms" % (
        int(bad.sum()), float(np.max(err - rnd) / scale))
    r_err, r_rnd = float(err.max() / scale), float(rnd.max() / scale)
    if r_rnd + 2 * FP32_BLOCK <= STATED_BAR:
        assert r_err <= STATED_BAR, "max|err|/rms %.4g above the stated bar" % r_err
    return r_err, r_rnd


def fp32_sum_bound(Xd: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """Bound on |fp32 sum - exact| for Y = X W^T summed in any order with
    fp32 products exact (bf16 inputs) or rounded (fp32 inputs):
    2 * K * 2^-24 * sum |x w|, per element."""
    K = Xd.shape[1]
    return 2.0 * K * 2.0 ** -24 * (np.abs(Xd) @ np.abs(Wd).T) + 1e-30
