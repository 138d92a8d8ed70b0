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
VARIANT_AUTO, VARIANT_GEMV, VARIANT_SPLITK, VARIANT_MFMA, VARIANT_ROWS = range(5)
OP_SKINNY_GEMM, OP_ROUTE, OP_EXPERT_FFN, OP_BLOCK, OP_ROUTE_LATENT = range(5)
KERNEL_ROUTE, KERNEL_EXPERT_UP, KERNEL_EXPERT_DOWN, KERNEL_COMBINE, KERNEL_SKINNY, KERNEL_BLOCK, KERNEL_STREAM = range(7)
VARIANTS = {"auto": VARIANT_AUTO, "gemv": VARIANT_GEMV, "splitk": VARIANT_SPLITK, "mfma": VARIANT_MFMA, "rows": VARIANT_ROWS}
SCHEDULE_AUTO, SCHEDULE_LAUNCHES, SCHEDULE_FUSED, SCHEDULE_ROUTER_IN_UP = range(4)
SCHEDULES = {"auto": SCHEDULE_AUTO, "launches": SCHEDULE_LAUNCHES, "fused": SCHEDULE_FUSED,
             "router_in_up": SCHEDULE_ROUTER_IN_UP}
SHARED_AUTO, SHARED_IN_UP, SHARED_IN_ROUTER = range(3)
SHARED_SCHEDULES = {"auto": SHARED_AUTO, "up": SHARED_IN_UP, "router": SHARED_IN_ROUTER}

# name: (restype, argtypes)
_P, _I, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "moe_abi_version": (_I, []),
    "moe_status_str": (ctypes.c_char_p, [_I]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_last_variant": (ctypes.c_char_p, []),
    "moe_set_variant": (_I, [_I]),
    "moe_set_block_schedule": (_I, [_I]),
    "moe_set_shared_schedule": (_I, [_I]),
    "moe_plan_words": (_I, [_I, _I, _I]),
    "moe_workspace_bytes": (_Z, [_I] * 10),
    "moe_workspace_init": (_I, [_P, _Z, _P]),
    "moe_workspace_status_offset": (_Z, []),
    "moe_stream_read": (_I, [_P, _Z, _P, _I, _P]),
    "moe_prefetch": (_I, [_I, _P, _P, _P, _I, _P]),
    "moe_profile_events": (_I, [_I, _P, _P]),
    "skinny_gemm": (_I, [_I, _I, _I, _I, _P, _P, _P, _I, _P, _Z, _P]),
    "skinny_gemm_residual": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _Z, _P]),
    "moe_route": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_route_latent": (_I, [_I] * 6 + [_P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _P, _P, _Z, _P]),
    "moe_expert_ffn": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _Z, _P]),
    "moe_combine": (_I, [_I, _I, _I, _I, _P, _P, _I, _P, _P]),
    "moe_block": (_I, [_I] * 7 + [_P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_block_streams": (_I, [_I] * 7 + [_P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P, _P, _P, _P]),
    "moe_block_noalloc": (_I, [_I] * 7 + [_P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
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


class _Args:
    """Argument validation before any C call: every tensor's shape, dtype and
    contiguity first, then that all of them sit on one GPU.  The C side gets
    only pointers and sizes, so a transposed view, a short weight array or a
    host tensor must never reach it."""

    def __init__(self):
        self.tensors = []

    def arr(self, name, t, shape, dtype, optional=False):
        if t is None:
            if optional:
                return None
            raise ValueError("%s is required" % name)
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s: a torch.Tensor expected, got %s" % (name, type(t).__name__))
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
        if t.dtype != dtype:
            raise TypeError("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        self.tensors.append((name, t))
        return t

    def workspace(self, ws, optional=False):
        if ws is None:
            if optional:
                return None
            raise ValueError("ws is required")
        if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1:
            raise TypeError("ws: a 1-D uint8 torch.Tensor expected")
        if not ws.is_contiguous():
            raise ValueError("ws must be contiguous")
        self.tensors.append(("ws", ws))
        return ws

    def on_gpu(self):
        dev = None
        for name, t in self.tensors:
            if t.device.type != "cuda":
                raise ValueError("%s must be in GPU memory (device %s)" % (name, t.device))
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError("%s is on %s, the other arguments on %s" % (name, t.device, dev))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dt(t) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError("a torch.Tensor expected, got %s" % type(t).__name__)
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype == torch.float32:
        return DT_F32
    raise TypeError("bf16 or fp32 tensors expected, got %s" % t.dtype)


def _shape(name, t, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s: a torch.Tensor expected, got %s" % (name, type(t).__name__))
    if t.dim() != ndim:
        raise ValueError("%s: %d dimensions expected, got shape %s" % (name, ndim, tuple(t.shape)))
    return tuple(t.shape)


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


def set_shared_schedule(name_or_id) -> int:
    v = SHARED_SCHEDULES[name_or_id] if isinstance(name_or_id, str) else int(name_or_id)
    return lib.moe_set_shared_schedule(v)


def plan_words(B: int, k: int, E: int) -> int:
    return lib.moe_plan_words(B, k, E)


def workspace_bytes(op: int, dtype: int, B=0, d=0, E=0, k=0, I=0, Is=0, N=0, K=0) -> int:
    return lib.moe_workspace_bytes(op, dtype, B, d, E, k, I, Is, N, K)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace of nbytes (rounded up to 256 B)."""
    return torch.zeros((nbytes + 255) // 256 * 256, dtype=torch.uint8, device=device)


def workspace_status(ws: torch.Tensor) -> int:
    """The fused schedule's barrier status word of ws (0: no barrier gave up).
    Reads device memory: synchronises with the device."""
    o = lib.moe_workspace_status_offset()
    return int(ws[o:o + 4].view(torch.int32).item())


def workspace_init(ws: torch.Tensor, stream=None):
    _check(lib.moe_workspace_init(_ptr(ws), ws.numel(), _stream(stream)))


def profile_events(kernel: int, start=None, stop=None):
    """Bracket every launch of `kernel` with the two events (torch.cuda.Event
    objects that have been recorded once, or raw hipEvent_t); None disarms."""
    h = lambda e: None if e is None else (e.cuda_event if hasattr(e, "cuda_event") else e)
    _check(lib.moe_profile_events(kernel, h(start), h(stop)))


def _gemm_args(X, W, Y, ws, R=None):
    B, K = _shape("X", X, 2)
    N, _ = _shape("W", W, 2)
    tdt = X.dtype
    a = _Args()
    a.arr("X", X, (B, K), tdt)
    a.arr("W", W, (N, K), tdt)
    if R is not None:
        a.arr("R", R, (B, N), tdt)
    _shape("Y", Y, 2)
    if Y.dtype not in (tdt, torch.float32):
        raise TypeError("Y: dtype %s, expected %s or torch.float32" % (Y.dtype, tdt))
    a.arr("Y", Y, (B, N), Y.dtype)
    a.workspace(ws, optional=True)
    a.on_gpu()
    return B, N, K


def skinny_gemm(X, W, Y, ws=None, stream=None):
    B, N, K = _gemm_args(X, W, Y, ws)
    _check(lib.skinny_gemm(_dt(X), B, N, K, _ptr(X), _ptr(W), _ptr(Y), _dt(Y), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream(stream)))


def skinny_gemm_residual(X, W, R, Y, ws=None, stream=None):
    if R is None:
        raise ValueError("R is required")
    B, N, K = _gemm_args(X, W, Y, ws, R)
    _check(lib.skinny_gemm_residual(_dt(X), B, N, K, _ptr(X), _ptr(W), _ptr(R), _ptr(Y), _dt(Y), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(stream)))


def _bias(a, bias, bias_ld, B, E):
    if bias is None:
        return
    if bias_ld == 0:
        a.arr("bias", bias, (E,), torch.float32)
    elif bias_ld == E:
        a.arr("bias", bias, (B, E), torch.float32)
    else:
        raise ValueError("bias_ld must be 0 (bias [E]) or E (bias [B][E]), got %d" % bias_ld)


def moe_route(X, Wr, k, topk_ids, topk_w, plan, ws, bias=None, bias_ld=0, logits_out=None,
              stream=None):
    B, d = _shape("X", X, 2)
    E, _ = _shape("Wr", Wr, 2)
    a = _Args()
    a.arr("X", X, (B, d), X.dtype)
    a.arr("Wr", Wr, (E, d), X.dtype)
    _bias(a, bias, bias_ld, B, E)
    a.arr("topk_ids", topk_ids, (B, k), torch.int32)
    a.arr("topk_w", topk_w, (B, k), torch.float32)
    a.arr("plan", plan, (plan_words(B, k, E),), torch.int32)
    a.arr("logits_out", logits_out, (B, E), torch.float32, optional=True)
    a.workspace(ws)
    a.on_gpu()
    _check(lib.moe_route(_dt(X), B, d, E, k, _ptr(X), _ptr(Wr), _ptr(bias), bias_ld,
                         _ptr(topk_ids), _ptr(topk_w), _ptr(plan), _ptr(logits_out), _ptr(ws),
                         ws.numel(), _stream(stream)))


def moe_route_latent(X, Wr, Wl, k, topk_ids, topk_w, plan, latent_out, ws, bias=None, bias_ld=0,
                     logits_out=None, stream=None):
    """moe_route with the latent input projection latent_out = X . Wl^T in the
    same product over X (latent_out of X's dtype or fp32)."""
    B, d = _shape("X", X, 2)
    E, _ = _shape("Wr", Wr, 2)
    L, _ = _shape("Wl", Wl, 2)
    a = _Args()
    a.arr("X", X, (B, d), X.dtype)
    a.arr("Wr", Wr, (E, d), X.dtype)
    a.arr("Wl", Wl, (L, d), X.dtype)
    _bias(a, bias, bias_ld, B, E)
    a.arr("topk_ids", topk_ids, (B, k), torch.int32)
    a.arr("topk_w", topk_w, (B, k), torch.float32)
    a.arr("plan", plan, (plan_words(B, k, E),), torch.int32)
    _shape("latent_out", latent_out, 2)
    if latent_out.dtype not in (X.dtype, torch.float32):
        raise TypeError("latent_out: dtype %s, expected %s or torch.float32" % (latent_out.dtype, X.dtype))
    a.arr("latent_out", latent_out, (B, L), latent_out.dtype)
    a.arr("logits_out", logits_out, (B, E), torch.float32, optional=True)
    a.workspace(ws)
    a.on_gpu()
    _check(lib.moe_route_latent(_dt(X), B, d, E, k, L, _ptr(X), _ptr(Wr), _ptr(Wl), _ptr(bias), bias_ld,
                                _ptr(topk_ids), _ptr(topk_w), _ptr(plan), _ptr(latent_out), _dt(latent_out),
                                _ptr(logits_out), _ptr(ws), ws.numel(), _stream(stream)))


def _experts(a, X, W13, W2, Ws13, Ws2):
    """Shapes of the expert weights against X [B][d]: (B, d, E, I, Is)."""
    B, d = _shape("X", X, 2)
    E, two_i, _ = _shape("W13", W13, 3)
    if two_i % 2:
        raise ValueError("W13: [E][2I][d] expected, got %s" % (tuple(W13.shape),))
    I = two_i // 2
    a.arr("X", X, (B, d), X.dtype)
    a.arr("W13", W13, (E, 2 * I, d), X.dtype)
    a.arr("W2", W2, (E, d, I), X.dtype)
    if (Ws13 is None) != (Ws2 is None):
        raise ValueError("Ws13 and Ws2 come together (both or neither)")
    Is = 0
    if Ws13 is not None:
        two_s, _ = _shape("Ws13", Ws13, 2)
        if two_s % 2:
            raise ValueError("Ws13: [2Is][d] expected, got %s" % (tuple(Ws13.shape),))
        Is = two_s // 2
        a.arr("Ws13", Ws13, (2 * Is, d), X.dtype)
        a.arr("Ws2", Ws2, (d, Is), X.dtype)
    return B, d, E, I, Is


def moe_expert_ffn(X, plan, W13, W2, k, Yslot, ws, Ws13=None, Ws2=None, stream=None):
    a = _Args()
    B, d, E, I, Is = _experts(a, X, W13, W2, Ws13, Ws2)
    a.arr("plan", plan, (plan_words(B, k, E),), torch.int32)
    a.arr("Yslot", Yslot, (B, k + 1, d), torch.float32)
    a.workspace(ws)
    a.on_gpu()
    _check(lib.moe_expert_ffn(_dt(X), B, d, E, k, I, _ptr(X), _ptr(plan), _ptr(W13),
                              _ptr(W2), Is, _ptr(Ws13), _ptr(Ws2), _ptr(Yslot), _ptr(ws),
                              ws.numel(), _stream(stream)))


def moe_combine(Yslot, topk_w, has_shared, out, stream=None):
    B, kp1, d = _shape("Yslot", Yslot, 3)
    a = _Args()
    a.arr("Yslot", Yslot, (B, kp1, d), torch.float32)
    a.arr("topk_w", topk_w, (B, kp1 - 1), torch.float32)
    _dt(out)
    a.arr("out", out, (B, d), out.dtype)
    a.on_gpu()
    _check(lib.moe_combine(_dt(out), B, d, kp1 - 1, _ptr(Yslot), _ptr(topk_w), int(bool(has_shared)),
                           _ptr(out), _stream(stream)))


def moe_block(X, Wr, k, W13, W2, out, ws, Ws13=None, Ws2=None, bias=None, bias_ld=0,
              topk_ids=None, topk_w=None, stream=None):
    a = _Args()
    B, d, E, I, Is = _experts(a, X, W13, W2, Ws13, Ws2)
    a.arr("Wr", Wr, (E, d), X.dtype)
    _bias(a, bias, bias_ld, B, E)
    a.arr("out", out, (B, d), X.dtype)
    a.arr("topk_ids", topk_ids, (B, k), torch.int32, optional=True)
    a.arr("topk_w", topk_w, (B, k), torch.float32, optional=True)
    a.workspace(ws)
    a.on_gpu()
    _check(lib.moe_block(_dt(X), B, d, E, k, I, Is, _ptr(X), _ptr(Wr), _ptr(bias), bias_ld,
                         _ptr(W13), _ptr(W2), _ptr(Ws13), _ptr(Ws2), _ptr(out), _ptr(topk_ids),
                         _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream)))


def _event(e):
    """Raw hipEvent_t of a torch.cuda.Event (recorded once, so that it exists)."""
    if hasattr(e, "cuda_event"):
        if not e.cuda_event:
            e.record()
        return e.cuda_event
    return e


def moe_block_streams(X, Wr, k, W13, W2, out, ws, side_stream, fork_event, join_event, Ws13=None, Ws2=None,
                      bias=None, bias_ld=0, topk_ids=None, topk_w=None, stream=None):
    """moe_block with the shared expert on side_stream (torch.cuda.Stream),
    ordered by fork_event / join_event (torch.cuda.Event objects)."""
    a = _Args()
    B, d, E, I, Is = _experts(a, X, W13, W2, Ws13, Ws2)
    a.arr("Wr", Wr, (E, d), X.dtype)
    _bias(a, bias, bias_ld, B, E)
    a.arr("out", out, (B, d), X.dtype)
    a.arr("topk_ids", topk_ids, (B, k), torch.int32, optional=True)
    a.arr("topk_w", topk_w, (B, k), torch.float32, optional=True)
    a.workspace(ws)
    a.on_gpu()
    _check(lib.moe_block_streams(_dt(X), B, d, E, k, I, Is, _ptr(X), _ptr(Wr), _ptr(bias), bias_ld,
                                 _ptr(W13), _ptr(W2), _ptr(Ws13), _ptr(Ws2), _ptr(out), _ptr(topk_ids),
                                 _ptr(topk_w), _ptr(ws), ws.numel(), _stream(stream), _stream(side_stream),
                                 _event(fork_event), _event(join_event)))


def moe_block_noalloc(X, Wr, k, W13, W2, out, Ws13=None, Ws2=None, bias=None, bias_ld=0,
                      topk_ids=None, topk_w=None, stream=None):
    """moe_block on the library's device-resident scratch (no workspace
    argument, nothing allocated); calls overlapping on one GPU race."""
    a = _Args()
    B, d, E, I, Is = _experts(a, X, W13, W2, Ws13, Ws2)
    a.arr("Wr", Wr, (E, d), X.dtype)
    _bias(a, bias, bias_ld, B, E)
    a.arr("out", out, (B, d), X.dtype)
    a.arr("topk_ids", topk_ids, (B, k), torch.int32, optional=True)
    a.arr("topk_w", topk_w, (B, k), torch.float32, optional=True)
    a.on_gpu()
    _check(lib.moe_block_noalloc(_dt(X), B, d, E, k, I, Is, _ptr(X), _ptr(Wr), _ptr(bias), bias_ld,
                                 _ptr(W13), _ptr(W2), _ptr(Ws13), _ptr(Ws2), _ptr(out), _ptr(topk_ids),
                                 _ptr(topk_w), _stream(stream)))


def stream_read(src, sink, stream=None):
    """The read-only streaming yardstick: reads all of src (any contiguous
    device tensor, byte size a multiple of 16) in sink.numel() workgroups;
    sink (uint32 as int32 [workgroups]) receives the XOR of each slice."""
    a = _Args()
    if not isinstance(src, torch.Tensor) or not src.is_contiguous():
        raise ValueError("src: a contiguous torch.Tensor expected")
    a.tensors.append(("src", src))
    _shape("sink", sink, 1)
    a.arr("sink", sink, tuple(sink.shape), torch.int32)
    a.on_gpu()
    _check(lib.moe_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), sink.numel(),
                               _stream(stream)))


def prefetch(tensors, sink, stream=None):
    """Cached reads of up to 8 contiguous device tensors (byte sizes multiples
    of 16) into L2 and the Infinity Cache, in sink.numel() workgroups; sink
    (int32 [workgroups]) receives the XOR of each workgroup's words."""
    a = _Args()
    tensors = [t for t in tensors if t is not None]
    if not 1 <= len(tensors) <= 8:
        raise ValueError("1 to 8 tensors expected, got %d" % len(tensors))
    for i, t in enumerate(tensors):
        if not isinstance(t, torch.Tensor) or not t.is_contiguous():
            raise ValueError("tensor %d: a contiguous torch.Tensor expected" % i)
        a.tensors.append(("tensor %d" % i, t))
    _shape("sink", sink, 1)
    a.arr("sink", sink, tuple(sink.shape), torch.int32)
    a.on_gpu()
    n = len(tensors)
    ptrs = (ctypes.c_void_p * n)(*[t.data_ptr() for t in tensors])
    sizes = (ctypes.c_size_t * n)(*[t.numel() * t.element_size() for t in tensors])
    _check(lib.moe_prefetch(n, ptrs, sizes, _ptr(sink), sink.numel(), _stream(stream)))
