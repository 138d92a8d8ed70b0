"""Seeded synthetic inputs for the decode MoE block and the dense skinny GEMM.

This module draws random numbers and encodes them; it holds none of the
block's arithmetic, and both the HIP path's tests and the CPU oracle take
their inputs from it.

Every array comes from its own numpy PCG64 stream keyed by
``(seed, tag, index...)`` so that any one expert's weights, or any one token's
activation row, can be drawn on its own and always comes out the same.
bf16 arrays are returned as ``uint16`` holding the raw bf16 bits, rounded from
fp32 draws to nearest-even; fp32 arrays as ``float32``.

Workloads (decode MoE block on one tensor-parallel weight shard):

* ``tiny``     fp32, B=1, d=1024, E=16, top-2, I=256, no shared expert.
* ``tp16_b1``  bf16, B=1, d=7168, E=384, top-8, I=Is=128.
* ``tp16_b8``  as ``tp16_b1`` at B=8, Gumbel noise added to the router logits.
* ``tp8_b64``  bf16, B=64, d=7168, E=384, top-8, I=Is=256, Zipf(1.1) log-prior
               over experts added to the router logits.
* dense skinny GEMM: X [B][7168] . W[3072][7168]^T, B in 1..64.

x ~ N(0, 1); every weight ~ N(0, 1/fan_in) with fan_in the shard's input
dimension (d for the router and gate/up rows, I or Is for the down rows).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

# stream tags
_T_X, _T_WR, _T_W13, _T_W2, _T_WS13, _T_WS2, _T_GUMBEL, _T_PERM = 1, 2, 3, 4, 5, 6, 7, 8
_T_DX, _T_DW = 9, 10
_T_OX, _T_OW, _T_OR = 11, 12, 13
_T_LAT = 14


@dataclass(frozen=True)
class MoEConfig:
    name: str
    B: int
    d: int
    E: int
    k: int
    I: int
    Is: int          # 0: no shared expert
    dtype: str       # "f32" or "bf16"
    routing: str     # "plain", "gumbel" or "zipf"
    zipf_s: float = 1.1

    def with_batch(self, B: int) -> "MoEConfig":
        return replace(self, B=B, name="%s@B%d" % (self.name, B))


CONFIGS = {
    "tiny": MoEConfig("tiny", 1, 1024, 16, 2, 256, 0, "f32", "plain"),
    "tp16_b1": MoEConfig("tp16_b1", 1, 7168, 384, 8, 128, 128, "bf16", "plain"),
    "tp16_b8": MoEConfig("tp16_b8", 8, 7168, 384, 8, 128, 128, "bf16", "gumbel"),
    "tp8_b64": MoEConfig("tp8_b64", 64, 7168, 384, 8, 256, 256, "bf16", "zipf"),
}

DENSE_N = 3072
DENSE_K = 7168
DENSE_BATCHES = (1, 2, 4, 8, 16, 32, 64)
# latent input projection concatenated with the router (the pages give no
# latent dimension): Wl [LATENT_L][d]
LATENT_L = 1024
# attention output projection with residual: back from one rank's attention
# width (taken equal to the input projection's share, 3072) to d = 7168
OPROJ_N = 7168
OPROJ_K = 3072


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(v) for v in key])


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _encode(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(a)
    raise ValueError(dtype)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


# ---- MoE block -------------------------------------------------------------

def x_row(cfg: MoEConfig, seed: int, t: int, attempt: int = 0) -> np.ndarray:
    """Token t's activation row; ``attempt`` > 0 gives an independent redraw."""
    return _encode(_normal(_rng(seed, _T_X, t, attempt), cfg.d, 1.0), cfg.dtype)


def x(cfg: MoEConfig, seed: int, attempts=None) -> np.ndarray:
    att = attempts if attempts is not None else [0] * cfg.B
    return np.stack([x_row(cfg, seed, t, att[t]) for t in range(cfg.B)])


def router_w(cfg: MoEConfig, seed: int) -> np.ndarray:
    return _encode(_normal(_rng(seed, _T_WR), (cfg.E, cfg.d), cfg.d ** -0.5), cfg.dtype)


def expert_w13(cfg: MoEConfig, seed: int, e: int) -> np.ndarray:
    """Fused [2I][d]: gate rows 0..I-1, then up rows I..2I-1."""
    return _encode(_normal(_rng(seed, _T_W13, e), (2 * cfg.I, cfg.d), cfg.d ** -0.5), cfg.dtype)


def expert_w2(cfg: MoEConfig, seed: int, e: int) -> np.ndarray:
    """Down projection [d][I]."""
    return _encode(_normal(_rng(seed, _T_W2, e), (cfg.d, cfg.I), cfg.I ** -0.5), cfg.dtype)


def shared_w13(cfg: MoEConfig, seed: int):
    if not cfg.Is:
        return None
    return _encode(_normal(_rng(seed, _T_WS13), (2 * cfg.Is, cfg.d), cfg.d ** -0.5), cfg.dtype)


def shared_w2(cfg: MoEConfig, seed: int):
    if not cfg.Is:
        return None
    return _encode(_normal(_rng(seed, _T_WS2), (cfg.d, cfg.Is), cfg.Is ** -0.5), cfg.dtype)


def gumbel_row(cfg: MoEConfig, seed: int, t: int, attempt: int = 0) -> np.ndarray:
    """Standard Gumbel noise -ln(-ln U), U ~ Uniform(0, 1), one row [E]."""
    u = _rng(seed, _T_GUMBEL, t, attempt).uniform(np.finfo(np.float64).tiny, 1.0, cfg.E)
    return (-np.log(-np.log(u))).astype(np.float32)


def zipf_prior(cfg: MoEConfig, seed: int) -> np.ndarray:
    """Per-expert log-prior -s * ln(rank), rank a seeded permutation of 1..E."""
    rank = _rng(seed, _T_PERM).permutation(cfg.E) + 1
    return (-cfg.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)


def bias(cfg: MoEConfig, seed: int, attempts=None):
    """(bias, bias_ld): None/0 for plain routing, [B][E]/E for Gumbel noise,
    [E]/0 for the Zipf prior."""
    if cfg.routing == "plain":
        return None, 0
    if cfg.routing == "gumbel":
        att = attempts if attempts is not None else [0] * cfg.B
        return np.stack([gumbel_row(cfg, seed, t, att[t]) for t in range(cfg.B)]), cfg.E
    if cfg.routing == "zipf":
        return zipf_prior(cfg, seed), 0
    raise ValueError(cfg.routing)


def all_expert_w13(cfg: MoEConfig, seed: int, experts=None) -> np.ndarray:
    """[E][2I][d]; experts not listed (if a list is given) are left zero."""
    out = np.zeros((cfg.E, 2 * cfg.I, cfg.d), np.float32 if cfg.dtype == "f32" else np.uint16)
    for e in (range(cfg.E) if experts is None else experts):
        out[e] = expert_w13(cfg, seed, e)
    return out


def all_expert_w2(cfg: MoEConfig, seed: int, experts=None) -> np.ndarray:
    out = np.zeros((cfg.E, cfg.d, cfg.I), np.float32 if cfg.dtype == "f32" else np.uint16)
    for e in (range(cfg.E) if experts is None else experts):
        out[e] = expert_w2(cfg, seed, e)
    return out


# ---- dense skinny GEMM ----------------------------------------------------

def dense_x(B: int, K: int = DENSE_K, seed: int = 0) -> np.ndarray:
    return to_bf16_bits(_normal(_rng(seed, _T_DX, B), (B, K), 1.0))


def dense_w(N: int = DENSE_N, K: int = DENSE_K, seed: int = 0) -> np.ndarray:
    return to_bf16_bits(_normal(_rng(seed, _T_DW), (N, K), K ** -0.5))


def oproj_x(B: int, K: int = OPROJ_K, seed: int = 0) -> np.ndarray:
    return to_bf16_bits(_normal(_rng(seed, _T_OX, B), (B, K), 1.0))


def oproj_w(N: int = OPROJ_N, K: int = OPROJ_K, seed: int = 0) -> np.ndarray:
    return to_bf16_bits(_normal(_rng(seed, _T_OW), (N, K), K ** -0.5))


def oproj_r(B: int, N: int = OPROJ_N, seed: int = 0) -> np.ndarray:
    """The residual stream entering the output projection: N(0, 1)."""
    return to_bf16_bits(_normal(_rng(seed, _T_OR, B), (B, N), 1.0))


def latent_w(cfg: MoEConfig, seed: int, L: int = LATENT_L) -> np.ndarray:
    """Latent input projection Wl [L][d] ~ N(0, 1/d)."""
    return _encode(_normal(_rng(seed, _T_LAT), (L, cfg.d), cfg.d ** -0.5), cfg.dtype)
