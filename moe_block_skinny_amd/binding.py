"""Thin ctypes binding of libmoe_skinny.so (the C ABI in include/moe_skinny.h).

Argument marshalling only: every function below passes device pointers,
sizes and the caller's current HIP stream straight to the C call of the same
name and raises MoeError on a non-OK status.  Torch tensors are used for
device memory and streams; no arithmetic of the block happens here, and there
is no fallback: if the library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_skinny.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = range(5)
DT_F32, DT_BF16 = 0, 1
VARIANT_AUTO, VARIANT_GEMV, VARIANT_SPLITK, VARIANT_MFMA = range(4)
OP_SKINNY_GEMM, OP_ROUTE, OP_EXPERT_FFN, OP_BLOCK = range(4)
KERNEL_ROUTE, KERNEL_EXPERT_UP, KERNEL_EXPERT_DOWN, KERNEL_COMBINE, KERNEL_SKINNY, KERNEL_BLOCK = range(6)
VARIANTS = {"auto": VARIANT_AUTO, "gemv": VARIANT_GEMV, "splitk": VARIANT_SPLITK, "mfma": VARIANT_MFMA}
SCHEDULE_AUTO, SCHEDULE_LAUNCHES, SCHEDULE_FUSED = range(3)
SCHEDULES = {"auto": SCHEDULE_AUTO, "launches": SCHEDULE_LAUNCHES, "fused": SCHEDULE_FUSED}

# name: (restype, argtypes)
_P, _I, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "moe_abi_version": (_I, []),
    "moe_status_str": (ctypes.c_char_p, [_I]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_last_variant": (ctypes.c_char_p, []),
    "moe_set_variant": (_I, [_I]),
    "moe_set_block_schedule": (_I, [_I]),
    "moe_plan_words": (_I, [_I, _I, _I]),
    "moe_workspace_bytes": (_Z, [_I] * 10),
    "moe_workspace_init": (_I, [_P, _Z, _P]),
    "moe_profile_events": (_I, [_I, _P, _P]),
    "skinny_gemm": (_I, [_I, _I, _I, _I, _P, _P, _P, _I, _P, _Z, _P]),
    "skinny_gemm_residual": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _Z, _P]),
    "moe_route": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_expert_ffn": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _Z, _P]),
    "moe_combine": (_I, [_I, _I, _I, _I, _P, _P, _I, _P, _P]),
    "moe_block": (_I, [_I] * 7 + [_P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
}


class MoeError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__("%s (status %d): %s" % (_name(status), status, detail))
        self.status = status


def _name(s):
    return {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_EUNSUPPORTED", 3: "MOE_EWORKSPACE", 4: "MOE_EHIP"}.get(s, "?")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError("libmoe_skinny.so is not built (run __graft_entry__.build() or "
                          "python -m moe_block_skinny_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = load()


def _check(status):
    if status != OK:
        raise MoeError(status, lib.moe_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return t                     # raw integer pointer (tests of validation)
    return t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype == torch.float32:
        return DT_F32
    raise TypeError("bf16 or fp32 tensors expected, got %s" % t.dtype)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def last_variant() -> str:
    return lib.moe_last_variant().decode()


def set_variant(name_or_id) -> int:
    v = VARIANTS[name_or_id] if isinstance(name_or_id, str) else int(name_or_id)
    return lib.moe_set_variant(v)


def set_block_schedule(name_or_id) -> int:
    v = SCHEDULES[name_or_id] if isinstance(name_or_id, str) else int(name_or_id)
    return lib.moe_set_block_schedule(v)


def plan_words(B: int, k: int, E: int) -> int:
    return lib.moe_plan_words(B, k, E)


def workspace_bytes(op: int, dtype: int, B=0, d=0, E=0, k=0, I=0, Is=0, N=0, K=0) -> int:
    return lib.moe_workspace_bytes(op, dtype, B, d, E, k, I, Is, N, K)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace of nbytes (rounded up to 256 B)."""
    return torch.zeros((nbytes + 255) // 256 * 256, dtype=torch.uint8, device=device)


def workspace_init(ws: torch.Tensor, stream=None):
    _check(lib.moe_workspace_init(_ptr(ws), ws.numel(), _stream(stream)))


def profile_events(kernel: int, start=None, stop=None):
    """Bracket every launch of `kernel` with the two events (torch.cuda.Event
    objects that have been recorded once, or raw hipEvent_t); None disarms."""
    h = lambda e: None if e is None else (e.cuda_event if hasattr(e, "cuda_event") else e)
    _check(lib.moe_profile_events(kernel, h(start), h(stop)))


def skinny_gemm(X, W, Y, ws=None, stream=None):
    B, K = X.shape
    N = W.shape[0]
    _check(lib.skinny_gemm(_dt(X), B, N, K, _ptr(X), _ptr(W), _ptr(Y), _dt(Y), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream(stream)))


def skinny_gemm_residual(X, W, R, Y, ws=None, stream=None):
    B, K = X.shape
    N = W.shape[0]
    _check(lib.skinny_gemm_residual(_dt(X), B, N, K, _ptr(X), _ptr(W), _ptr(R), _ptr(Y), _dt(Y), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(stream)))


def moe_route(X, Wr, k, topk_ids, topk_w, plan, ws, bias=None, bias_ld=0, logits_out=None,
              stream=None):
    B, d = X.shape
    E = Wr.shape[0]
    _check(lib.moe_route(_dt(X), B, d, E, k, _ptr(X), _ptr(Wr), _ptr(bias), bias_ld,
                         _ptr(topk_ids), _ptr(topk_w), _ptr(plan), _ptr(logits_out), _ptr(ws),
                         ws.numel(), _stream(stream)))


def moe_expert_ffn(X, plan, W13, W2, k, Yslot, ws, Ws13=None, Ws2=None, stream=None):
    B, d = X.shape
    E, two_i, _ = W13.shape
    Is = 0 if Ws13 is None else Ws13.shape[0] // 2
    _check(lib.moe_expert_ffn(_dt(X), B, d, E, k, two_i // 2, _ptr(X), _ptr(plan), _ptr(W13),
                              _ptr(W2), Is, _ptr(Ws13), _ptr(Ws2), _ptr(Yslot), _ptr(ws),
                              ws.numel(), _stream(stream)))


def moe_combine(Yslot, topk_w, has_shared, out, stream=None):
    B, kp1, d = Yslot.shape
    _check(lib.moe_combine(_dt(out), B, d, kp1 - 1, _ptr(Yslot), _ptr(topk_w), int(bool(has_shared)),
                           _ptr(out), _stream(stream)))


def moe_block(X, Wr, k, W13, W2, out, ws, Ws13=None, Ws2=None, bias=None, bias_ld=0,
              topk_ids=None, topk_w=None, stream=None):
    B, d = X.shape
    E, two_i, _ = W13.shape
    Is = 0 if Ws13 is None else Ws13.shape[0] // 2
    _check(lib.moe_block(_dt(X), B, d, E, k, two_i // 2, Is, _ptr(X), _ptr(Wr), _ptr(bias), bias_ld,
                         _ptr(W13), _ptr(W2), _ptr(Ws13), _ptr(Ws2), _ptr(out), _ptr(topk_ids),
                         _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream)))
