"""ctypes wrapper around oracle.c, the plain CPU definition of the MoE block.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.

Arrays follow the numpy conventions of the input generator: bf16 data is a
``uint16`` array holding the raw bf16 bits, fp32 data is ``float32``.  Results
come back as float64 (int32 for ids and plans).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

DT_F32 = 0
DT_BF16 = 1


_LIB_OMP = os.path.join(_HERE, "liboracle_omp.so")
_lib_omp = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction): the plain
    single-thread library, and the same source with OpenMP (tokens of a block
    in parallel) for the all-cores CPU timing."""
    for lib, extra in ((_LIB, []), (_LIB_OMP, ["-fopenmp"])):
        if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
            tmp = lib + ".tmp%d" % os.getpid()
            subprocess.run(
                ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                 "-shared", "-fPIC"] + extra + ["-o", tmp, _SRC, "-lm"],
                check=True,
            )
            os.replace(tmp, lib)
    return _LIB


def _declare(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_skinny_gemm.argtypes = [I, I, I, I, P, P, P]
    lib.oracle_skinny_gemm_residual.argtypes = [I, I, I, I, P, P, P, P]
    lib.oracle_router_logits.argtypes = [I, I, I, I, P, P, P, I, P]
    lib.oracle_topk.argtypes = [I, I, P, P, P]
    lib.oracle_plan_words.restype = I
    lib.oracle_plan_words.argtypes = [I, I, I]
    lib.oracle_plan.argtypes = [I, I, I, P, P]
    lib.oracle_route.argtypes = [I, I, I, I, I, P, P, P, I, P, P, P, P]
    lib.oracle_expert.argtypes = [I, I, I, P, ctypes.c_size_t, P, P, P, P]
    lib.oracle_moe_block.restype = I
    lib.oracle_moe_block.argtypes = [I] * 7 + [P, P, P, I, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_combine.argtypes = [I, I, I, P, P, I, P]
    lib.oracle_latent_projection.argtypes = [I, I, I, I, P, P, P]
    lib.oracle_threads.restype = I
    lib.oracle_threads.argtypes = []
    return lib


def _load(parallel: bool = False):
    global _lib, _lib_omp
    with _lock:
        if _lib is None:
            build()
            _lib = _declare(ctypes.CDLL(_LIB))
            _lib_omp = _declare(ctypes.CDLL(_LIB_OMP))
    return _lib_omp if parallel else _lib


def threads(parallel: bool = False) -> int:
    """Threads the oracle's block runs its tokens on (1 for the plain build)."""
    return _load(parallel).oracle_threads()


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.float32:
        return DT_F32
    raise TypeError("oracle inputs are uint16 (bf16 bits) or float32, got %s" % a.dtype)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def silu(z: float) -> float:
    return _load().oracle_silu(float(z))


def plan_words(B: int, k: int, E: int) -> int:
    return _load().oracle_plan_words(B, k, E)


def skinny_gemm(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Y[b][n] = sum_c X[b][c] W[n][c] in fp64."""
    X, W = _c(X), _c(W)
    B, K = X.shape
    N = W.shape[0]
    assert W.shape[1] == K and _dt(X) == _dt(W)
    Y = np.empty((B, N), np.float64)
    _load().oracle_skinny_gemm(_dt(X), B, N, K, _p(X), _p(W), _p(Y))
    return Y


def skinny_gemm_residual(X: np.ndarray, W: np.ndarray, R: np.ndarray) -> np.ndarray:
    """Y[b][n] = sum_c X[b][c] W[n][c] + R[b][n] in fp64 (R of X's dtype)."""
    X, W, R = _c(X), _c(W), _c(R)
    B, K = X.shape
    N = W.shape[0]
    assert W.shape[1] == K and R.shape == (B, N) and _dt(X) == _dt(W) == _dt(R)
    Y = np.empty((B, N), np.float64)
    _load().oracle_skinny_gemm_residual(_dt(X), B, N, K, _p(X), _p(W), _p(R), _p(Y))
    return Y


def router_logits(X, Wr, bias=None, bias_ld=0) -> np.ndarray:
    X, Wr, bias = _c(X), _c(Wr), _c(bias, np.float32)
    B, d = X.shape
    E = Wr.shape[0]
    L = np.empty((B, E), np.float64)
    _load().oracle_router_logits(_dt(X), B, d, E, _p(X), _p(Wr), _p(bias), bias_ld, _p(L))
    return L


def topk(logits_row: np.ndarray, k: int):
    """ids (ascending) and weights of the top-k of one token's logits."""
    row = _c(logits_row, np.float64)
    ids = np.empty(k, np.int32)
    w = np.empty(k, np.float64)
    _load().oracle_topk(row.shape[0], k, _p(row), _p(ids), _p(w))
    return ids, w


def plan(ids: np.ndarray, E: int) -> np.ndarray:
    ids = _c(ids, np.int32)
    B, k = ids.shape
    out = np.empty(plan_words(B, k, E), np.int32)
    _load().oracle_plan(B, k, E, _p(ids), _p(out))
    return out


def route(X, Wr, k, bias=None, bias_ld=0):
    """(logits [B][E], ids [B][k], w [B][k], plan) for the router stage."""
    X, Wr, bias = _c(X), _c(Wr), _c(bias, np.float32)
    B, d = X.shape
    E = Wr.shape[0]
    L = np.empty((B, E), np.float64)
    ids = np.empty((B, k), np.int32)
    w = np.empty((B, k), np.float64)
    pl = np.empty(plan_words(B, k, E), np.int32)
    _load().oracle_route(_dt(X), B, d, E, k, _p(X), _p(Wr), _p(bias), bias_ld,
                         _p(L), _p(ids), _p(w), _p(pl))
    return L, ids, w, pl


def expert(x_row, W13, W2):
    """(y [d], h [I]) of one expert on one token."""
    x_row, W13, W2 = _c(x_row), _c(W13), _c(W2)
    d = x_row.shape[-1]
    I = W13.shape[0] // 2
    y = np.empty(d, np.float64)
    h = np.empty(I, np.float64)
    _load().oracle_expert(_dt(x_row), d, I, _p(x_row), 0, _p(W13), _p(W2), _p(y), _p(h))
    return y, h


def latent_projection(X, Wl) -> np.ndarray:
    """Latent input projection latent = X . Wl^T: X [B][d], Wl [L][d] ->
    float64 [B][L]."""
    X, Wl = _c(X), _c(Wl)
    B, d = X.shape
    L = Wl.shape[0]
    out = np.empty((B, L), np.float64)
    _load().oracle_latent_projection(_dt(X), B, d, L, _p(X), _p(Wl), _p(out))
    return out


def moe_block(X, Wr, k, W13e, W2e, Ws13=None, Ws2=None, bias=None, bias_ld=0, parallel=False):
    """Whole block.  W13e / W2e: sequences of E per-expert arrays (or None for
    experts no token selects).  Returns a dict with logits, ids, w, plan,
    yslot [B][k+1][d] and out [B][d].  parallel: the OpenMP build (tokens on
    all cores; same arithmetic per token)."""
    X, Wr, bias = _c(X), _c(Wr), _c(bias, np.float32)
    Ws13, Ws2 = _c(Ws13), _c(Ws2)
    B, d = X.shape
    E = Wr.shape[0]
    keep = []
    p13 = (ctypes.c_void_p * E)()
    p2 = (ctypes.c_void_p * E)()
    I = None
    for e in range(E):
        if W13e[e] is not None:
            a, b = _c(W13e[e]), _c(W2e[e])
            keep += [a, b]
            p13[e] = a.ctypes.data
            p2[e] = b.ctypes.data
            I = a.shape[0] // 2
    Is = 0 if Ws13 is None else Ws13.shape[0] // 2
    L = np.empty((B, E), np.float64)
    ids = np.empty((B, k), np.int32)
    w = np.empty((B, k), np.float64)
    pl = np.empty(plan_words(B, k, E), np.int32)
    ys = np.empty((B, k + 1, d), np.float64)
    out = np.empty((B, d), np.float64)
    rc = _load(parallel).oracle_moe_block(
        _dt(X), B, d, E, k, I or 0, Is, _p(X), _p(Wr), _p(bias), bias_ld,
        ctypes.cast(p13, ctypes.c_void_p), ctypes.cast(p2, ctypes.c_void_p),
        _p(Ws13), _p(Ws2), _p(L), _p(ids), _p(w), _p(pl), _p(ys), _p(out))
    if rc != 0:
        raise ValueError("a selected expert has no weights")
    return dict(logits=L, ids=ids, w=w, plan=pl, yslot=ys, out=out)


def combine(yslot_f32, w_f32, has_shared: bool) -> np.ndarray:
    ys, w = _c(yslot_f32, np.float32), _c(w_f32, np.float32)
    B, kp1, d = ys.shape
    out = np.empty((B, d), np.float64)
    _load().oracle_combine(B, d, kp1 - 1, _p(ys), _p(w), int(bool(has_shared)), _p(out))
    return out
