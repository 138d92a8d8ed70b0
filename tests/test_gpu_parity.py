"""GPU parity of every C-ABI call against the CPU oracle (needs an MI355X).

Bars (derived in the design doc):
  * integer, index and plan outputs: bit-exact;
  * small-integer inputs (every sum exact in fp32): bit-exact floats too;
  * fp32 sums: within 2 * K * 2^-24 * sum|x w| of the oracle (fp64);
  * bf16 outputs: that plus bf16 rounding, 2^-8 * |ref|;
  * gate weights: 1e-5 absolute; per-slot expert outputs: 2e-4 * rms;
  * block output (bf16): per element |err| <= |bf16(ref) - ref| + 2e-3 rms,
    and max|err| <= 2e-2 * rms(ref), the stated bar, wherever rounding the
    exact result to bf16 leaves room for it (every workload here).
Shapes span several row blocks and ragged tails; forced kernel shapes run at
every batch each one supports, so every path is exercised.
"""
import contextlib

import numpy as np
import pytest
import torch

from moe_block_skinny_amd import binding as mb
from moe_block_skinny_amd import synth
from oracle import oracle as orc
from tests import inputs
from tests.gpu_util import check_block_output, dev, host, widen, rms, say, fp32_sum_bound

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def variant(name):
    prev = mb.set_variant(name)
    try:
        yield
    finally:
        mb.set_variant(prev)


def bf16_of_ints(a):
    return synth.to_bf16_bits(np.asarray(a, np.float32))


def ws_for(op, dtype, **kw):
    return mb.workspace(mb.workspace_bytes(op, dtype, **kw))


SHAPES = {"gemv": [1, 2], "splitk": [1, 2, 3, 4, 5, 8], "mfma": [1, 2, 5, 9, 16, 17, 33, 64], "rows": [1, 2, 3, 4, 5, 7, 8],
          "auto": [1, 2, 3, 4, 5, 6, 8, 16, 24, 48, 64]}


# ---------------------------------------------------------------- skinny_gemm

@pytest.mark.parametrize("var", ["auto", "gemv", "splitk", "mfma", "rows"])
@pytest.mark.parametrize("K", [7168, 1056, 256])
def test_skinny_gemm_integer_exact(var, K):
    rng = np.random.default_rng(K)
    N = 200
    Wi = rng.integers(-3, 4, (N, K))
    W = dev(bf16_of_ints(Wi))
    for B in SHAPES[var]:
        say("skinny_gemm integer", var, "B", B, "K", K)
        Xi = rng.integers(-3, 4, (B, K))
        ref = (Xi @ Wi.T).astype(np.float64)
        X = dev(bf16_of_ints(Xi))
        Y = torch.full((B, N), float("nan"), device="cuda")
        ws = ws_for(mb.OP_SKINNY_GEMM, mb.DT_BF16, B=B, N=N, K=K)
        with variant(var):
            mb.skinny_gemm(X, W, Y, ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(Y), ref), (var, B)
        if var != "auto":
            assert var in mb.last_variant()


@pytest.mark.parametrize("B", synth.DENSE_BATCHES)
def test_skinny_gemm_dense_workload(B):
    """Attention input projection workload: N=3072, K=7168, bf16."""
    Xh, Wh = synth.dense_x(B), synth.dense_w()
    ref = orc.skinny_gemm(Xh, Wh)
    bound = fp32_sum_bound(widen(Xh), widen(Wh))
    X, W = dev(Xh), dev(Wh)
    N, K = Wh.shape
    ws = ws_for(mb.OP_SKINNY_GEMM, mb.DT_BF16, B=B, N=N, K=K)
    for var in ["auto"] + [v for v in ("gemv", "splitk", "mfma", "rows") if B in SHAPES[v] or v == "mfma"]:
        say("skinny_gemm dense", var, "B", B)
        Y32 = torch.empty((B, N), device="cuda")
        Y16 = torch.empty((B, N), device="cuda", dtype=torch.bfloat16)
        with variant(var):
            mb.skinny_gemm(X, W, Y32, ws)
            mb.skinny_gemm(X, W, Y16, ws)
        torch.cuda.synchronize()
        err = np.abs(host(Y32) - ref)
        assert np.all(err <= bound), (var, B, float(err.max()))
        err16 = np.abs(host(Y16) - ref)
        assert np.all(err16 <= bound + 2.0 ** -8 * np.abs(ref)), (var, B)


@pytest.mark.parametrize("var", ["auto", "gemv", "splitk", "mfma", "rows"])
@pytest.mark.parametrize("K", [3072, 1056])
def test_skinny_gemm_residual_integer_exact(var, K):
    """Output projection with residual on small integers: every sum is exact
    in fp32, so every kernel shape must give X W^T + R bit for bit."""
    rng = np.random.default_rng(K)
    N = synth.OPROJ_N
    Wi = rng.integers(-3, 4, (N, K))
    W = dev(bf16_of_ints(Wi))
    for B in SHAPES[var][:4] + ([64] if var in ("auto", "mfma") else []):
        Xi = rng.integers(-3, 4, (B, K))
        Ri = rng.integers(-50, 51, (B, N))
        ref = (Xi @ Wi.T + Ri).astype(np.float64)
        Y = torch.full((B, N), float("nan"), device="cuda")
        ws = ws_for(mb.OP_SKINNY_GEMM, mb.DT_BF16, B=B, N=N, K=K)
        with variant(var):
            mb.skinny_gemm_residual(dev(bf16_of_ints(Xi)), W, dev(bf16_of_ints(Ri)), Y, ws)
        torch.cuda.synchronize()
        say("skinny_gemm_residual integer", var, "B", B, "K", K)
        assert np.array_equal(host(Y), ref), (var, B)


@pytest.mark.parametrize("B", [1, 2, 8, 64])
def test_skinny_gemm_residual_workload(B):
    """Output projection workload (N = 7168, K = 3072, bf16) against the
    oracle; the in-place form (Y is R) gives the same bits."""
    Xh, Wh, Rh = synth.oproj_x(B), synth.oproj_w(), synth.oproj_r(B)
    ref = orc.skinny_gemm_residual(Xh, Wh, Rh)
    bound = fp32_sum_bound(widen(Xh), widen(Wh)) + 2.0 ** -23 * np.abs(widen(Rh))
    N, K = Wh.shape
    X, W, R = dev(Xh), dev(Wh), dev(Rh)
    ws = ws_for(mb.OP_SKINNY_GEMM, mb.DT_BF16, B=B, N=N, K=K)
    Y32 = torch.empty((B, N), device="cuda")
    Y16 = torch.empty((B, N), device="cuda", dtype=torch.bfloat16)
    mb.skinny_gemm_residual(X, W, R, Y32, ws)
    mb.skinny_gemm_residual(X, W, R, Y16, ws)
    Rin = R.clone()
    mb.skinny_gemm_residual(X, W, Rin, Rin, ws)
    torch.cuda.synchronize()
    say("skinny_gemm_residual workload B", B, mb.last_variant())
    err = np.abs(host(Y32) - ref)
    assert np.all(err <= bound), float(err.max())
    assert np.all(np.abs(host(Y16) - ref) <= bound + 2.0 ** -8 * np.abs(ref))
    assert torch.equal(Rin.view(torch.int16), Y16.view(torch.int16))


def test_skinny_gemm_workspace_reuse():
    """Back-to-back MFMA products with K slices over ONE workspace, with
    different inputs and batch sizes: every call's partial sums must be read
    as that call wrote them, never as an earlier call left them in a cache."""
    N, K = 3072, 7168
    Wh = synth.dense_w()
    W = dev(Wh)
    ws = ws_for(mb.OP_SKINNY_GEMM, mb.DT_BF16, B=64, N=N, K=K)
    outs = []
    with variant("mfma"):
        for i, B in enumerate((64, 32, 17, 64, 16, 48, 33, 64)):
            Xh = synth.to_bf16_bits(np.random.default_rng(100 + i).standard_normal((B, K)).astype(np.float32))
            Y = torch.empty((B, N), device="cuda")
            mb.skinny_gemm(dev(Xh), W, Y, ws)
            outs.append((Xh, Y))
    torch.cuda.synchronize()
    for i, (Xh, Y) in enumerate(outs):
        ref = orc.skinny_gemm(Xh, Wh)
        bound = fp32_sum_bound(widen(Xh), widen(Wh))
        err = np.abs(host(Y) - ref)
        assert np.all(err <= bound), (i, Xh.shape[0], float(err.max()))


def test_skinny_gemm_fp32():
    rng = np.random.default_rng(3)
    for B, N, K in [(1, 70, 1024), (2, 33, 260), (7, 129, 516)]:
        say("skinny_gemm fp32", B, N, K)
        Xh = rng.standard_normal((B, K)).astype(np.float32)
        Wh = rng.standard_normal((N, K)).astype(np.float32)
        ref = orc.skinny_gemm(Xh, Wh)
        Y = torch.empty((B, N), device="cuda")
        ws = ws_for(mb.OP_SKINNY_GEMM, mb.DT_F32, B=B, N=N, K=K)
        mb.skinny_gemm(dev(Xh), dev(Wh), Y, ws)
        torch.cuda.synchronize()
        assert np.all(np.abs(host(Y) - ref) <= fp32_sum_bound(widen(Xh), widen(Wh)) + 1e-6 * np.abs(ref))


# ---------------------------------------------------------------- moe_route

def run_route(Xh, Wrh, k, bias=None, bias_ld=0):
    B, d = Xh.shape
    E = Wrh.shape[0]
    dt = mb.DT_BF16 if Xh.dtype == np.uint16 else mb.DT_F32
    ids = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((B, k), float("nan"), device="cuda")
    plan = torch.full((mb.plan_words(B, k, E),), -7, dtype=torch.int32, device="cuda")
    lo = torch.full((B, E), float("nan"), device="cuda")
    ws = ws_for(mb.OP_ROUTE, dt, B=B, d=d, E=E, k=k)
    mb.moe_route(dev(Xh), dev(Wrh), k, ids, w, plan, ws,
                 bias=None if bias is None else dev(bias), bias_ld=bias_ld, logits_out=lo)
    torch.cuda.synchronize()
    return host(ids), host(w), host(plan), host(lo)


@pytest.mark.parametrize("var", ["auto", "gemv", "splitk", "mfma"])
def test_route_integer_ties(var):
    """Small-integer logits: exact sums and many exact ties, so logits, the
    lower-index tie-break, ids and plan must all match bit for bit."""
    rng = np.random.default_rng(21)
    E, d, k = 384, 7168, 8
    Wi = rng.integers(-1, 2, (E, d)) * (rng.random((E, d)) < 0.01)
    for B in SHAPES[var]:
        say("route integer", var, "B", B)
        Xi = rng.integers(-2, 3, (B, d))
        Xh, Wh = bf16_of_ints(Xi), bf16_of_ints(Wi)
        L, ids, w, pl = orc.route(Xh, Wh, k)
        with variant(var):
            g_ids, g_w, g_pl, g_l = run_route(Xh, Wh, k)
        assert np.array_equal(g_l, L)
        assert np.array_equal(g_ids, ids)
        assert np.array_equal(g_pl, pl)
        assert np.max(np.abs(g_w - w)) <= 1e-6


@pytest.mark.parametrize("name", ["tiny", "tp16_b1", "tp16_b8", "tp8_b64"])
def test_route_workloads(name):
    c = inputs.case(name)
    say("route workload", name, "redraws", c.redraws)
    variants = ["auto"] + [v for v in ("gemv", "splitk", "mfma")
                           if c.cfg.B in SHAPES[v] and not (v == "mfma" and c.cfg.dtype == "f32")]
    bound = fp32_sum_bound(widen(c.X), widen(c.Wr)) + 2.0 ** -23 * np.abs(c.logits)
    for var in variants:
        say("route workload", name, var)
        with variant(var):
            g_ids, g_w, g_pl, g_l = run_route(c.X, c.Wr, c.cfg.k, c.bias, c.bias_ld)
        assert np.all(np.abs(g_l - c.logits) <= bound), var
        assert np.array_equal(g_ids, c.ids), var
        assert np.array_equal(g_pl, c.plan), var
        assert np.max(np.abs(g_w - c.w)) <= 1e-5, var


def test_route_exact_ties_uniform():
    """All logits equal: the k lowest expert ids win with weight 1/k."""
    d, E, k = 1024, 40, 8
    Xh = bf16_of_ints(np.ones((3, d)))
    Wh = bf16_of_ints(np.zeros((E, d)))
    g_ids, g_w, g_pl, _ = run_route(Xh, Wh, k)
    assert np.array_equal(g_ids, np.tile(np.arange(k), (3, 1)))
    assert np.all(g_w == 1.0 / k)
    assert np.array_equal(g_pl, orc.plan(g_ids.astype(np.int32), E))


# ---------------------------------------------------------------- expert FFN

def integer_experts(rng, E, d, I, x_ones=64):
    """Gate rows give g in [40, 59] (silu(g) == g exactly in fp32 and fp64),
    sparse up rows keep |h| < 2^11, so every stage is exact."""
    W13 = np.zeros((E, 2 * I, d), np.int64)
    for e in range(E):
        for i in range(I):
            W13[e, i, :40 + (i + e) % 20] = 1
            cols = rng.choice(d, 16, replace=False)
            W13[e, I + i, cols] = rng.choice([-1, 1], 16)
    W2 = rng.integers(-1, 2, (E, d, I))
    return W13, W2


@pytest.mark.parametrize("var", ["auto", "gemv", "mfma"])
def test_expert_ffn_integer_exact(var):
    rng = np.random.default_rng(5)
    E, d, k, I, Is = 16, 1024, 4, 64, 96
    W13i, W2i = integer_experts(rng, E, d, I)
    Ws13i, Ws2i = integer_experts(rng, 1, d, Is)
    W13, W2 = dev(bf16_of_ints(W13i)), dev(bf16_of_ints(W2i))
    Ws13, Ws2 = dev(bf16_of_ints(Ws13i[0])), dev(bf16_of_ints(Ws2i[0]))
    for B in ([1, 3, 8] if var == "gemv" else [1, 3, 8, 20, 64]):
        say("expert integer", var, "B", B)
        Xi = rng.integers(-2, 3, (B, d))
        Xi[:, :64] = 1
        ids = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(B)]).astype(np.int32)
        plan = orc.plan(ids, E)
        Xh = bf16_of_ints(Xi)
        Y = torch.full((B, k + 1, d), float("nan"), device="cuda")
        ws = ws_for(mb.OP_EXPERT_FFN, mb.DT_BF16, B=B, d=d, E=E, k=k, I=I, Is=Is)
        ws.view(torch.float32).fill_(float("nan"))       # no counters in the FFN workspace
        with variant(var):
            mb.moe_expert_ffn(dev(Xh), dev(plan), W13, W2, k, Y, ws, Ws13, Ws2)
        torch.cuda.synchronize()
        g = host(Y)
        for t in range(B):
            for j in range(k):
                e = ids[t, j]
                y, _ = orc.expert(Xh[t], bf16_of_ints(W13i[e]), bf16_of_ints(W2i[e]))
                assert np.array_equal(g[t, j], y), (var, B, t, j)
            ys, _ = orc.expert(Xh[t], bf16_of_ints(Ws13i[0]), bf16_of_ints(Ws2i[0]))
            assert np.array_equal(g[t, k], ys), (var, B, t)


def gpu_weights(c):
    """Full [E] weight tensors with every expert the routing does not select
    filled with NaN, so reading one shows up in the result."""
    cfg = c.cfg
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    W13 = torch.full((cfg.E, 2 * cfg.I, cfg.d), float("nan"), dtype=tdt, device="cuda")
    W2 = torch.full((cfg.E, cfg.d, cfg.I), float("nan"), dtype=tdt, device="cuda")
    for e in c.touched:
        W13[e] = dev(c.W13[e])
        W2[e] = dev(c.W2[e])
    Ws13 = None if c.Ws13 is None else dev(c.Ws13)
    Ws2 = None if c.Ws2 is None else dev(c.Ws2)
    return W13, W2, Ws13, Ws2


_wcache = {}


def case_and_weights(name):
    if name not in _wcache:
        _wcache.clear()
        c = inputs.case(name)
        _wcache[name] = (c, gpu_weights(c))
    return _wcache[name]


@pytest.mark.parametrize("name", ["tiny", "tp16_b1", "tp16_b8", "tp8_b64"])
def test_expert_ffn_workloads(name):
    c, (W13, W2, Ws13, Ws2) = case_and_weights(name)
    cfg = c.cfg
    ref = c.oracle_block()["yslot"]
    has_s = Ws13 is not None
    cols = cfg.k + 1 if has_s else cfg.k
    scale = rms(ref[:, :cols])
    variants = ["auto"] + (["gemv"] if cfg.B <= 8 else []) + (["mfma"] if cfg.dtype == "bf16" else [])
    dt = mb.DT_BF16 if cfg.dtype == "bf16" else mb.DT_F32
    for var in variants:
        say("expert workload", name, var)
        Y = torch.full((cfg.B, cfg.k + 1, cfg.d), float("nan"), device="cuda")
        ws = ws_for(mb.OP_EXPERT_FFN, dt, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k, I=cfg.I, Is=cfg.Is)
        ws.view(torch.float32).fill_(float("nan"))
        with variant(var):
            mb.moe_expert_ffn(dev(c.X), dev(c.plan), W13, W2, cfg.k, Y, ws, Ws13, Ws2)
        torch.cuda.synchronize()
        g = host(Y)[:, :cols]
        assert np.all(np.isfinite(g)), var
        err = np.max(np.abs(g - ref[:, :cols]))
        say("  max|err|/rms", err / scale)
        assert err <= 2e-4 * scale, (var, err / scale)


# ---------------------------------------------------------------- combine

@pytest.mark.parametrize("dt,B,d,k,shared", [("bf16", 1, 7168, 8, True), ("bf16", 64, 7168, 8, False),
                                             ("f32", 1, 1024, 2, False), ("bf16", 5, 96, 3, True)])
def test_combine(dt, B, d, k, shared):
    rng = np.random.default_rng(B * 100 + d)
    ys = rng.standard_normal((B, k + 1, d)).astype(np.float32)
    w = rng.uniform(0, 1, (B, k)).astype(np.float32)
    ref = orc.combine(ys, w, shared)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = torch.full((B, d), float("nan"), dtype=tdt, device="cuda")
    mb.moe_combine(dev(ys), dev(w), shared, out)
    torch.cuda.synchronize()
    g = host(out)
    bound = 4 * (k + 1) * 2.0 ** -24 * (np.abs(ys[:, :k]).astype(np.float64) * w[:, :, None]).sum(1) + np.abs(ys[:, k]) * (2.0 ** -23)
    if dt == "bf16":
        bound = bound + 2.0 ** -8 * np.abs(ref)
    assert np.all(np.abs(g - ref) <= bound + 1e-30)


# ---------------------------------------------------------------- whole block

def run_block(c, W13, W2, Ws13, Ws2, ws=None):
    cfg = c.cfg
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dt = mb.DT_BF16 if cfg.dtype == "bf16" else mb.DT_F32
    out = torch.full((cfg.B, cfg.d), float("nan"), dtype=tdt, device="cuda")
    ids = torch.full((cfg.B, cfg.k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((cfg.B, cfg.k), float("nan"), device="cuda")
    if ws is None:
        ws = ws_for(mb.OP_BLOCK, dt, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k, I=cfg.I, Is=cfg.Is)
    bias = None if c.bias is None else dev(c.bias)
    mb.moe_block(dev(c.X), dev(c.Wr), cfg.k, W13, W2, out, ws, Ws13, Ws2, bias, c.bias_ld, ids, w)
    torch.cuda.synchronize()
    assert mb.workspace_status(ws) == 0   # no in-launch wait gave up
    return out, ids, w


@pytest.mark.parametrize("name", ["tiny", "tp16_b1", "tp16_b8", "tp8_b64"])
def test_block_workloads(name):
    c, (W13, W2, Ws13, Ws2) = case_and_weights(name)
    ref = c.oracle_block()
    say("block workload", name, "distinct experts", len(c.touched), "redraws", c.redraws)
    out, ids, w = run_block(c, W13, W2, Ws13, Ws2)
    g = host(out)
    assert np.array_equal(host(ids), c.ids)
    assert np.max(np.abs(host(w) - c.w)) <= 1e-5
    assert np.all(np.isfinite(g))
    if c.cfg.dtype == "bf16":
        r_err, r_rnd = check_block_output(g, ref["out"])
        say("  max|err|/rms(out) %.5f, exact result rounded to bf16: %.5f" % (r_err, r_rnd))
        assert r_rnd + 2e-3 <= 2e-2    # the stated bar applies to every workload and was asserted
    else:
        scale = rms(ref["out"])
        err = np.max(np.abs(g - ref["out"]))
        say("  max|err|/rms(out)", err / scale)
        assert err <= 1e-4 * scale


@pytest.mark.parametrize("name", ["tp16_b1", "tp16_b8"])
def test_block_equals_composed_calls_and_is_deterministic(name):
    c, (W13, W2, Ws13, Ws2) = case_and_weights(name)
    cfg = c.cfg
    out1, _, _ = run_block(c, W13, W2, Ws13, Ws2)
    out2, _, _ = run_block(c, W13, W2, Ws13, Ws2)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    ids = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.B, cfg.k), device="cuda")
    plan = torch.empty((mb.plan_words(cfg.B, cfg.k, cfg.E),), dtype=torch.int32, device="cuda")
    ws = ws_for(mb.OP_ROUTE, mb.DT_BF16, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k)
    bias = None if c.bias is None else dev(c.bias)
    mb.moe_route(dev(c.X), dev(c.Wr), cfg.k, ids, w, plan, ws, bias=bias, bias_ld=c.bias_ld)
    Y = torch.empty((cfg.B, cfg.k + 1, cfg.d), device="cuda")
    wsf = ws_for(mb.OP_EXPERT_FFN, mb.DT_BF16, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k, I=cfg.I, Is=cfg.Is)
    mb.moe_expert_ffn(dev(c.X), plan, W13, W2, cfg.k, Y, wsf, Ws13, Ws2)
    out3 = torch.empty((cfg.B, cfg.d), dtype=torch.bfloat16, device="cuda")
    mb.moe_combine(Y, w, True, out3)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))


@pytest.mark.parametrize("B,k,E,I,dt", [(2, 8, 64, 64, "bf16"), (3, 6, 96, 64, "bf16"), (16, 4, 128, 64, "bf16"),
                                        (64, 1, 384, 64, "bf16"), (64, 1, 16, 64, "bf16"), (24, 8, 384, 128, "bf16"),
                                        (8, 1, 2, 4, "f32")])
def test_block_per_token_selection(B, k, E, I, dt):
    """Small-batch schedule (vector shape, B*k <= 64): from batch 2 each
    token's top-k is selected once, by one gate/up workgroup, and every
    workgroup waits for all tokens before it plans: ids bit-exact, weights
    within 1e-5, output within the bar, the status word clear, and a second
    call on the same workspace gives the same bits (the router launch clears
    the words the selections publish).  The fp32 case (E = 2 at B = 8) has
    fewer gate/up tasks than tokens, where the launch still needs one
    workgroup per token.  The bf16 cases above batch 8 take the matrix
    schedule (router slices, finish launch, plan from the ids) at the same
    small sizes."""
    cfg = synth.MoEConfig("select_b%d_k%d_e%d" % (B, k, E), B, 1024, E, k, I, 0 if dt == "f32" else I, dt, "gumbel")
    c = inputs.Case(cfg)
    W13, W2, Ws13, Ws2 = gpu_weights(c)
    ref = c.oracle_block()
    dtc = mb.DT_BF16 if dt == "bf16" else mb.DT_F32
    ws = ws_for(mb.OP_BLOCK, dtc, B=B, d=cfg.d, E=E, k=k, I=cfg.I, Is=cfg.Is)
    out1, ids1, w1 = run_block(c, W13, W2, Ws13, Ws2, ws=ws)
    out2, ids2, _ = run_block(c, W13, W2, Ws13, Ws2, ws=ws)
    say("per-token selection B=%d k=%d E=%d %s:" % (B, k, E, dt), mb.last_variant())
    assert np.array_equal(host(ids1), c.ids) and np.array_equal(host(ids2), c.ids)
    assert np.max(np.abs(host(w1) - c.w)) <= 1e-5
    if dt == "bf16":
        check_block_output(host(out1), ref["out"])
        assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    else:
        assert np.max(np.abs(host(out1) - ref["out"])) <= 1e-4 * rms(ref["out"])
        assert torch.equal(out1, out2)


def test_block_batch_invariance_on_gpu():
    """Token t's output at batch 8 equals its output run alone (the GPU may
    pick another kernel shape at B=1, so compare within the stated bar and
    require identical expert ids)."""
    c, (W13, W2, Ws13, Ws2) = case_and_weights("tp16_b8")
    out8, ids8, _ = run_block(c, W13, W2, Ws13, Ws2)
    g8 = host(out8)
    for t in (0, 5):
        sub = inputs.Case.__new__(inputs.Case)
        sub.cfg = c.cfg.with_batch(1)
        sub.X = c.X[t:t + 1]
        sub.Wr = c.Wr
        sub.bias = None if c.bias is None else c.bias[t:t + 1]
        sub.bias_ld = c.bias_ld
        out1, ids1, _ = run_block(sub, W13, W2, Ws13, Ws2)
        assert np.array_equal(host(ids1)[0], host(ids8)[t])
        assert np.max(np.abs(host(out1)[0] - g8[t])) <= 2e-2 * rms(g8[t])


def test_one_workspace_serves_every_op_in_turn():
    """One zero-filled workspace, sized for the biggest call, used in turn by
    a sliced MFMA product, the standalone router, experts and combine, and the
    block at two batch sizes: no call's data may land on another call's
    counters, so every block result equals the one on a fresh workspace."""
    cases = {n: case_and_weights(n) for n in ("tp8_b64", "tp16_b1")}
    nbytes = 0
    for c, _ in cases.values():
        cfg = c.cfg
        kw = dict(B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k, I=cfg.I, Is=cfg.Is)
        nbytes = max(nbytes, mb.workspace_bytes(mb.OP_BLOCK, mb.DT_BF16, **kw),
                     mb.workspace_bytes(mb.OP_ROUTE, mb.DT_BF16, **kw),
                     mb.workspace_bytes(mb.OP_EXPERT_FFN, mb.DT_BF16, **kw))
    nbytes = max(nbytes, mb.workspace_bytes(mb.OP_SKINNY_GEMM, mb.DT_BF16, B=64, N=3072, K=7168))
    ws = mb.workspace(nbytes)
    fresh = {n: run_block(c, *w)[0] for n, (c, w) in cases.items()}
    gen = torch.Generator(device="cuda").manual_seed(5)
    X = torch.randn((64, 7168), generator=gen, device="cuda").to(torch.bfloat16)
    W = (torch.randn((3072, 7168), generator=gen, device="cuda") * 0.01).to(torch.bfloat16)
    Y = torch.empty((64, 3072), dtype=torch.bfloat16, device="cuda")
    for name in ("tp8_b64", "tp16_b1", "tp8_b64"):
        c, (W13, W2, Ws13, Ws2) = cases[name]
        cfg = c.cfg
        mb.skinny_gemm(X, W, Y, ws)
        ids = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device="cuda")
        tw = torch.empty((cfg.B, cfg.k), device="cuda")
        plan = torch.empty((mb.plan_words(cfg.B, cfg.k, cfg.E),), dtype=torch.int32, device="cuda")
        bias = None if c.bias is None else dev(c.bias)
        mb.moe_route(dev(c.X), dev(c.Wr), cfg.k, ids, tw, plan, ws, bias=bias, bias_ld=c.bias_ld)
        Ys = torch.empty((cfg.B, cfg.k + 1, cfg.d), device="cuda")
        mb.moe_expert_ffn(dev(c.X), plan, W13, W2, cfg.k, Ys, ws, Ws13, Ws2)
        out = torch.empty((cfg.B, cfg.d), dtype=torch.bfloat16, device="cuda")
        mb.moe_combine(Ys, tw, True, out)
        got, got_ids, _ = run_block(c, W13, W2, Ws13, Ws2, ws=ws)
        say("shared workspace", name)
        assert np.array_equal(host(ids), c.ids)
        assert np.array_equal(host(got_ids), c.ids)
        assert torch.equal(got.view(torch.int16), fresh[name].view(torch.int16))
