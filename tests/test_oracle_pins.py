"""Pins of the CPU oracle against what mathematics fixes (no GPU).

The oracle is the reference the HIP path is judged by, so it is checked here
against things that do not come from the oracle itself: numpy's float64 and
int64 matrix products, brute force over every k-subset on tiny inputs,
closed forms (identity-like and permutation weights, huge gates where
silu(g) = g exactly), invariances (batch, expert relabelling, unselected
logits) and a hand-derived worked example.  Each group is chosen so that a
dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one test.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as orc
from moe_block_skinny_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def widen(a):
    """bf16 bits (uint16) or float32 -> float64, exactly."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def silu_ref(z):
    # logistic via tanh: sigma(z) = (1 + tanh(z/2)) / 2, independent of exp form
    return z * 0.5 * (1.0 + np.tanh(0.5 * z))


# ---------------------------------------------------------------- GEMM pins

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("B,N,K", [(1, 5, 24), (3, 17, 40), (7, 33, 264)])
def test_gemm_matches_numpy_float64(dt, B, N, K):
    rng = np.random.default_rng(B * 1000 + N)
    X = rng.standard_normal((B, K)).astype(np.float32)
    W = rng.standard_normal((N, K)).astype(np.float32)
    if dt == "bf16":
        X, W = synth.to_bf16_bits(X), synth.to_bf16_bits(W)
    Y = orc.skinny_gemm(X, W)
    ref = widen(X) @ widen(W).T
    bound = 2 * K * 2.0 ** -53 * (np.abs(widen(X)) @ np.abs(widen(W)).T) + 1e-300
    assert Y.shape == (B, N)
    assert np.all(np.abs(Y - ref) <= bound)


@pytest.mark.parametrize("splits", [1, 2, 4, 7, 16])
def test_gemm_integer_exact_and_split_k(splits):
    """Small-integer inputs: every sum is exact, so the oracle must equal the
    int64 product bit for bit, and summing K-split parts equals unsplit."""
    rng = np.random.default_rng(splits)
    B, N, K = 5, 19, 7168
    Xi = rng.integers(-3, 4, (B, K))
    Wi = rng.integers(-3, 4, (N, K))
    X = synth.to_bf16_bits(Xi.astype(np.float32))
    W = synth.to_bf16_bits(Wi.astype(np.float32))
    Y = orc.skinny_gemm(X, W)
    assert np.array_equal(Y, (Xi @ Wi.T).astype(np.float64))
    edges = np.linspace(0, K, splits + 1).astype(int)
    parts = sum(orc.skinny_gemm(np.ascontiguousarray(X[:, a:b]), np.ascontiguousarray(W[:, a:b]))
                for a, b in zip(edges[:-1], edges[1:]))
    assert np.array_equal(parts, Y)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gemm_residual_pins(dt):
    """Output projection with residual: numpy's float64 X W^T + R; a zero
    residual gives the plain product bit for bit; zero weights give R itself;
    integer inputs are exact (int64 product plus residual); a residual with
    rows swapped moves only those rows (R is indexed [b][n], not [n][b])."""
    rng = np.random.default_rng(11)
    B, N, K = 4, 37, 96
    X = rng.standard_normal((B, K)).astype(np.float32)
    W = rng.standard_normal((N, K)).astype(np.float32)
    R = rng.standard_normal((B, N)).astype(np.float32)
    if dt == "bf16":
        X, W, R = synth.to_bf16_bits(X), synth.to_bf16_bits(W), synth.to_bf16_bits(R)
    Y = orc.skinny_gemm_residual(X, W, R)
    ref = widen(X) @ widen(W).T + widen(R)
    bound = 2 * K * 2.0 ** -53 * (np.abs(widen(X)) @ np.abs(widen(W)).T + np.abs(widen(R))) + 1e-300
    assert np.all(np.abs(Y - ref) <= bound)
    assert np.array_equal(orc.skinny_gemm_residual(X, W, np.zeros_like(R)), orc.skinny_gemm(X, W))
    assert np.array_equal(orc.skinny_gemm_residual(X, np.zeros_like(W), R), widen(R))
    Rs = np.ascontiguousarray(R[::-1])
    Ys = orc.skinny_gemm_residual(X, W, Rs)
    assert np.allclose(Ys - orc.skinny_gemm(X, W), widen(Rs), rtol=0, atol=1e-12)
    Xi, Wi, Ri = rng.integers(-3, 4, (B, K)), rng.integers(-3, 4, (N, K)), rng.integers(-50, 51, (B, N))
    f = (lambda a: synth.to_bf16_bits(a.astype(np.float32))) if dt == "bf16" else (lambda a: a.astype(np.float32))
    assert np.array_equal(orc.skinny_gemm_residual(f(Xi), f(Wi), f(Ri)), (Xi @ Wi.T + Ri).astype(np.float64))


@pytest.mark.parametrize("bias_mode", ["none", "row", "per_token"])
def test_router_logits(bias_mode):
    rng = np.random.default_rng(7)
    B, d, E = 4, 64, 12
    X = synth.to_bf16_bits(rng.standard_normal((B, d)).astype(np.float32))
    Wr = synth.to_bf16_bits(rng.standard_normal((E, d)).astype(np.float32))
    bias, ld = None, 0
    ref = widen(X) @ widen(Wr).T
    if bias_mode == "row":
        bias = rng.standard_normal(E).astype(np.float32)
        ref = ref + bias.astype(np.float64)[None, :]
    elif bias_mode == "per_token":
        bias, ld = rng.standard_normal((B, E)).astype(np.float32), E
        ref = ref + bias.astype(np.float64)
    L = orc.router_logits(X, Wr, bias, ld)
    assert np.allclose(L, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- top-k pins

def _brute_topk(logits, k):
    """Among all k-subsets maximizing the sum of logits, the lexicographically
    smallest sorted index tuple."""
    best, best_set = None, None
    for S in itertools.combinations(range(len(logits)), k):
        s = sum(float(np.float32(logits[i])) for i in S)
        if best is None or s > best:
            best, best_set = s, S
    return list(best_set)


@pytest.mark.parametrize("E,k", [(4, 1), (6, 2), (9, 3), (12, 4), (12, 1)])
def test_topk_brute_force_distinct(E, k):
    rng = np.random.default_rng(E * 10 + k)
    for _ in range(40):
        logits = rng.standard_normal(E)
        ids, w = orc.topk(logits, k)
        assert list(ids) == _brute_topk(logits, k)


@pytest.mark.parametrize("E,k", [(6, 2), (9, 3), (12, 4)])
def test_topk_brute_force_ties(E, k):
    rng = np.random.default_rng(E + k)
    for _ in range(40):
        logits = rng.integers(-2, 3, E).astype(np.float64)   # many exact ties
        ids, w = orc.topk(logits, k)
        assert list(ids) == _brute_topk(logits, k)


def test_topk_weights_properties():
    rng = np.random.default_rng(3)
    E, k = 16, 4
    for _ in range(50):
        logits = rng.standard_normal(E) * 3
        ids, w = orc.topk(logits, k)
        assert np.all(np.diff(ids) > 0)
        assert abs(w.sum() - 1.0) <= 4 * k * 2.0 ** -52
        assert np.all(w > 0)
        # weight order follows logit order
        lf = logits.astype(np.float32).astype(np.float64)[ids]
        assert np.array_equal(np.argsort(-w, kind="stable"), np.argsort(-lf, kind="stable"))
        # equal to a softmax over all E renormalised over the selection
        p = np.exp(lf - lf.max())
        full = np.exp(logits.astype(np.float32).astype(np.float64) - logits.max())
        full = full / full.sum()
        ren = full[ids] / full[ids].sum()
        assert np.allclose(w, ren, rtol=1e-13, atol=0)
        assert np.allclose(w, p / p.sum(), rtol=1e-13, atol=0)
        # unselected logits do not move the weights at all
        thr = lf.min()
        l2 = logits.copy()
        mask = np.ones(E, bool)
        mask[ids] = False
        l2[mask] = np.minimum(l2[mask], thr) - rng.uniform(0.5, 5.0, mask.sum())
        ids2, w2 = orc.topk(l2, k)
        assert np.array_equal(ids, ids2) and np.array_equal(w, w2)


def test_topk_uniform_logits():
    ids, w = orc.topk(np.zeros(10), 4)
    assert list(ids) == [0, 1, 2, 3]
    assert np.all(w == 0.25)


def test_topk_decision_in_fp32():
    """Two logits that differ only below fp32 resolution tie, and the lower
    index wins, as it does for the GPU's fp32 logits."""
    l = np.array([1.0, 1.0 + 1e-12, 0.0])
    ids, _ = orc.topk(l, 1)
    assert list(ids) == [0]


# ---------------------------------------------------------------- plan pins

@pytest.mark.parametrize("B,k,E", [(1, 2, 16), (8, 8, 384), (64, 8, 384), (5, 3, 4)])
def test_plan(B, k, E):
    rng = np.random.default_rng(B * 7 + E)
    ids = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(B)]).astype(np.int32)
    pl = orc.plan(ids, E)
    maxa = min(E, B * k)
    n = pl[0]
    active = pl[1:1 + maxa]
    offs = pl[1 + maxa:2 + 2 * maxa]
    slots = pl[2 + 2 * maxa:]
    uniq = np.unique(ids)
    assert n == len(uniq)
    assert np.array_equal(active[:n], uniq) and np.all(active[n:] == -1)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")          # by expert, then slot
    assert np.array_equal(slots, order)
    counts = np.bincount(flat, minlength=E)[uniq]
    assert np.array_equal(np.diff(offs[:n + 1]), counts)
    assert offs[0] == 0 and offs[n] == B * k and np.all(offs[n:] == B * k)
    assert sorted(slots.tolist()) == list(range(B * k))


# ---------------------------------------------------------------- SiLU pins

def test_silu_closed_forms():
    assert orc.silu(0.0) == 0.0
    for z in np.linspace(-30, 30, 121):
        s = orc.silu(z)
        assert abs(s - silu_ref(z)) <= 1e-15 * max(1.0, abs(z))
        assert abs((s - orc.silu(-z)) - z) <= 1e-14 * max(1.0, abs(z))
    assert orc.silu(40.0) == 40.0            # 1 + exp(-40) == 1 in fp64


# ---------------------------------------------------------------- expert pins

def _perm_matrix(rows, cols, idx, scale=1.0):
    m = np.zeros((rows, cols), np.float32)
    m[np.arange(rows), idx] = scale
    return m


def test_expert_permutation_weights():
    """Gate = a*P, up = Q, down = R (non-symmetric permutations):
    y = R (silu(a P x) * (Q x)), by index arithmetic."""
    rng = np.random.default_rng(11)
    d, I, a = 48, 32, 1.7
    x = rng.standard_normal(d).astype(np.float32)
    p, q = rng.permutation(d)[:I], rng.permutation(d)[:I]
    rho = rng.integers(0, I, d)
    W13 = np.concatenate([_perm_matrix(I, d, p, a), _perm_matrix(I, d, q)])
    W2 = _perm_matrix(d, I, rho)
    y, h = orc.expert(x, W13, W2)
    xd = x.astype(np.float64)
    h_ref = silu_ref(np.float64(np.float32(a)) * xd[p]) * xd[q]
    assert np.allclose(h, h_ref, rtol=1e-14, atol=1e-300)
    assert np.allclose(y, h_ref[rho], rtol=1e-14, atol=1e-300)


def test_expert_integer_exact():
    """Gates forced to >= 40 so silu(g) == g in fp64; then the whole FFN is
    integer arithmetic and must equal the int64 computation exactly."""
    rng = np.random.default_rng(5)
    d, I = 256, 16
    x = rng.integers(-2, 3, d)
    x[:64] = 1
    Wg = np.zeros((I, d), np.int64)
    for i in range(I):
        Wg[i, :40 + i] = 1                       # g_i = 40 + i (x[:64] == 1)
    Wu = rng.integers(-2, 3, (I, d))
    W2 = rng.integers(-2, 3, (d, I))
    g = Wg @ x
    assert np.all(g >= 40)
    h = g * (Wu @ x)
    y_ref = W2 @ h
    enc = lambda a: synth.to_bf16_bits(np.asarray(a, np.float32))
    y, hh = orc.expert(enc(x), enc(np.concatenate([Wg, Wu])), enc(W2))
    assert np.array_equal(hh, h.astype(np.float64))
    assert np.array_equal(y, y_ref.astype(np.float64))


def test_expert_zero_gate_and_scaling():
    rng = np.random.default_rng(6)
    d, I = 64, 16
    x = rng.standard_normal(d).astype(np.float32)
    W13 = rng.standard_normal((2 * I, d)).astype(np.float32)
    W2 = rng.standard_normal((d, I)).astype(np.float32)
    Z = W13.copy()
    Z[:I] = 0
    y0, h0 = orc.expert(x, Z, W2)
    assert np.all(h0 == 0) and np.all(y0 == 0)
    y1, _ = orc.expert(x, W13, W2)
    y4, _ = orc.expert(x, W13, W2 * np.float32(4.0))
    assert np.array_equal(y4, 4.0 * y1)          # power-of-two scale is exact


# ---------------------------------------------------------------- block pins

def _rand_block(rng, B, d, E, k, I, Is, dt="f32"):
    enc = (lambda a: a.astype(np.float32)) if dt == "f32" else synth.to_bf16_bits
    X = enc(rng.standard_normal((B, d)).astype(np.float32))
    Wr = enc(rng.standard_normal((E, d)).astype(np.float32) / np.sqrt(d))
    W13 = [enc(rng.standard_normal((2 * I, d)).astype(np.float32) / np.sqrt(d)) for _ in range(E)]
    W2 = [enc(rng.standard_normal((d, I)).astype(np.float32) / np.sqrt(I)) for _ in range(E)]
    Ws13 = enc(rng.standard_normal((2 * Is, d)).astype(np.float32) / np.sqrt(d)) if Is else None
    Ws2 = enc(rng.standard_normal((d, Is)).astype(np.float32) / np.sqrt(Is)) if Is else None
    return X, Wr, W13, W2, Ws13, Ws2


def test_block_single_expert():
    rng = np.random.default_rng(1)
    X, Wr, W13, W2, Ws13, Ws2 = _rand_block(rng, 3, 32, 1, 1, 16, 8)
    r = orc.moe_block(X, Wr, 1, W13, W2, Ws13, Ws2)
    assert np.all(r["ids"] == 0) and np.all(r["w"] == 1.0)
    for t in range(3):
        y, _ = orc.expert(X[t], W13[0], W2[0])
        ys, _ = orc.expert(X[t], Ws13, Ws2)
        assert np.allclose(r["out"][t], y + ys, rtol=0, atol=1e-12)


def test_block_identical_experts():
    """All experts equal: out = FFN(x) + shared(x) whatever the routing."""
    rng = np.random.default_rng(2)
    B, d, E, k, I = 4, 40, 6, 3, 8
    X, Wr, W13, W2, Ws13, Ws2 = _rand_block(rng, B, d, E, k, I, 8)
    W13 = [W13[0]] * E
    W2 = [W2[0]] * E
    r = orc.moe_block(X, Wr, k, W13, W2, Ws13, Ws2)
    for t in range(B):
        y, _ = orc.expert(X[t], W13[0], W2[0])
        ys, _ = orc.expert(X[t], Ws13, Ws2)
        assert np.allclose(r["out"][t], y + ys, rtol=1e-13, atol=1e-13)


def test_block_zero_routed_down_is_shared_only():
    rng = np.random.default_rng(4)
    B, d, E, k, I = 3, 24, 5, 2, 8
    X, Wr, W13, W2, Ws13, Ws2 = _rand_block(rng, B, d, E, k, I, 8)
    W2 = [np.zeros_like(w) for w in W2]
    r = orc.moe_block(X, Wr, k, W13, W2, Ws13, Ws2)
    for t in range(B):
        ys, _ = orc.expert(X[t], Ws13, Ws2)
        assert np.array_equal(r["out"][t], ys)


def test_block_matches_numpy_composition():
    """Whole block against an independent numpy formulation (matrix products,
    argsort-based top-k, tanh-based silu)."""
    rng = np.random.default_rng(9)
    B, d, E, k, I, Is = 5, 64, 10, 3, 16, 8
    X, Wr, W13, W2, Ws13, Ws2 = _rand_block(rng, B, d, E, k, I, Is, "bf16")
    bias = rng.standard_normal((B, E)).astype(np.float32)
    r = orc.moe_block(X, Wr, k, W13, W2, Ws13, Ws2, bias, E)
    Xd = widen(X)
    L = Xd @ widen(Wr).T + bias
    Lf = L.astype(np.float32).astype(np.float64)
    for t in range(B):
        sel = np.sort(np.argsort(-Lf[t], kind="stable")[:k])
        assert np.array_equal(r["ids"][t], sel)
        p = np.exp(Lf[t, sel] - Lf[t, sel].max())
        w = p / p.sum()
        out = np.zeros(d)
        for j, e in enumerate(sel):
            W = widen(W13[e])
            h = silu_ref(W[:I] @ Xd[t]) * (W[I:] @ Xd[t])
            out += w[j] * (widen(W2[e]) @ h)
        Ws = widen(Ws13)
        out += widen(Ws2) @ (silu_ref(Ws[:Is] @ Xd[t]) * (Ws[Is:] @ Xd[t]))
        assert np.allclose(r["out"][t], out, rtol=1e-11, atol=1e-12)


def test_block_batch_invariance():
    rng = np.random.default_rng(12)
    B, d, E, k, I = 6, 32, 8, 2, 8
    X, Wr, W13, W2, Ws13, Ws2 = _rand_block(rng, B, d, E, k, I, 8)
    r = orc.moe_block(X, Wr, k, W13, W2, Ws13, Ws2)
    for t in range(B):
        r1 = orc.moe_block(X[t:t + 1], Wr, k, W13, W2, Ws13, Ws2)
        assert np.array_equal(r1["out"][0], r["out"][t])
        assert np.array_equal(r1["ids"][0], r["ids"][t])


def test_block_expert_relabelling():
    rng = np.random.default_rng(13)
    B, d, E, k, I = 5, 32, 9, 3, 8
    X, Wr, W13, W2, Ws13, Ws2 = _rand_block(rng, B, d, E, k, I, 8)
    bias = rng.standard_normal(E).astype(np.float32)
    r = orc.moe_block(X, Wr, k, W13, W2, Ws13, Ws2, bias, 0)
    perm = rng.permutation(E)            # new label i holds old expert perm[i]
    r2 = orc.moe_block(X, Wr[perm], k,
                       [W13[p] for p in perm], [W2[p] for p in perm], Ws13, Ws2,
                       bias[perm], 0)
    for t in range(B):
        assert np.array_equal(np.sort(perm[r2["ids"][t]]), r["ids"][t])
    assert np.allclose(r2["out"], r["out"], rtol=0, atol=1e-12 * np.sqrt(np.mean(r["out"] ** 2)))


def test_combine_stage():
    rng = np.random.default_rng(14)
    B, d, k = 3, 16, 4
    ys = rng.standard_normal((B, k + 1, d)).astype(np.float32)
    w = rng.uniform(0, 1, (B, k)).astype(np.float32)
    out = orc.combine(ys, w, True)
    ref = np.einsum("tj,tjd->td", w.astype(np.float64), ys[:, :k].astype(np.float64)) + ys[:, k]
    assert np.allclose(out, ref, rtol=1e-14, atol=1e-14)
    out0 = orc.combine(ys, w, False)
    assert np.allclose(out0, ref - ys[:, k], rtol=1e-13, atol=1e-13)


def test_hand_worked_example():
    """A block small enough to work by hand; values and derivation are in
    tests/golden/hand_example.json."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    f32 = lambda a: np.asarray(a, np.float32)
    r = orc.moe_block(f32(g["x"]), f32(g["Wr"]), g["k"], [f32(w) for w in g["W13"]],
                      [f32(w) for w in g["W2"]], f32(g["Ws13"]), f32(g["Ws2"]))
    assert r["ids"].tolist() == g["ids"]
    e = math.e
    w_ref = [1 / (1 + e), e / (1 + e)]
    assert np.allclose(r["w"][0], w_ref, rtol=1e-15, atol=0)
    s = lambda z: z / (1 + math.exp(-z))
    out_ref = [eval(expr, {"s": s, "e": e}) for expr in g["out_closed_form"]]
    assert np.allclose(r["out"][0], out_ref, rtol=1e-14, atol=1e-15)


def test_parallel_build_gives_the_same_bits():
    """The OpenMP build (tokens of the block on all cores, used for the
    all-cores CPU timing) computes every token with the same arithmetic as
    the plain build, so the two agree bit for bit."""
    cfg = synth.MoEConfig("omp", 6, 256, 12, 3, 32, 32, "bf16", "gumbel")
    X, Wr = synth.x(cfg, 4), synth.router_w(cfg, 4)
    bias, ld = synth.bias(cfg, 4)
    W13 = [synth.expert_w13(cfg, 4, e) for e in range(cfg.E)]
    W2 = [synth.expert_w2(cfg, 4, e) for e in range(cfg.E)]
    Ws13, Ws2 = synth.shared_w13(cfg, 4), synth.shared_w2(cfg, 4)
    a = orc.moe_block(X, Wr, cfg.k, W13, W2, Ws13, Ws2, bias, ld)
    b = orc.moe_block(X, Wr, cfg.k, W13, W2, Ws13, Ws2, bias, ld, parallel=True)
    assert orc.threads(False) == 1 and orc.threads(True) >= 1
    for key in ("logits", "ids", "w", "plan", "yslot", "out"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_latent_projection_pins(dt):
    """Latent input projection: against numpy float64 on random inputs
    (within the fp64 sum bound), bit-exact on small integers, K-split parts
    summing to the unsplit product, and a permutation matrix gathering the
    input columns it names."""
    rng = np.random.default_rng(31)
    B, d, L = 3, 96, 40
    X = rng.standard_normal((B, d)).astype(np.float32)
    Wl = rng.standard_normal((L, d)).astype(np.float32)
    if dt == "bf16":
        X, Wl = synth.to_bf16_bits(X), synth.to_bf16_bits(Wl)
    Y = orc.latent_projection(X, Wl)
    ref = widen(X) @ widen(Wl).T
    assert Y.shape == (B, L)
    assert np.all(np.abs(Y - ref) <= 2 * d * 2.0 ** -53 * (np.abs(widen(X)) @ np.abs(widen(Wl)).T) + 1e-300)
    Xi, Wi = rng.integers(-3, 4, (B, 2048)), rng.integers(-3, 4, (L, 2048))
    Xb, Wb = synth.to_bf16_bits(Xi.astype(np.float32)), synth.to_bf16_bits(Wi.astype(np.float32))
    Yi = orc.latent_projection(Xb, Wb)
    assert np.array_equal(Yi, (Xi @ Wi.T).astype(np.float64))
    parts = sum(orc.latent_projection(np.ascontiguousarray(Xb[:, a:a + 512]), np.ascontiguousarray(Wb[:, a:a + 512]))
                for a in range(0, 2048, 512))
    assert np.array_equal(parts, Yi)
    cols = rng.permutation(d)[:L]
    P = np.zeros((L, d), np.float32)
    P[np.arange(L), cols] = 1.0
    Pe = P if dt == "f32" else synth.to_bf16_bits(P)
    assert np.array_equal(orc.latent_projection(X, Pe), widen(X)[:, cols])
