"""moe_route_latent -- the router with the latent input projection in the
same product over x -- against the CPU oracle (needs an MI355X).

Small-integer inputs make every sum exact, so logits, the latent projection,
ids and plan must all be bit-exact on every kernel shape (the vector shapes
and the matrix shape with its K slices).  On the workloads' inputs the ids,
weights and plan match the oracle's routing and the latent projection is
within the fp32 sum bound (plus bf16 rounding when stored as bf16).  Ragged
cases: a latent block that fills one 16-row tile, an E and a d that leave
partial row groups."""
import contextlib

import numpy as np
import pytest
import torch

from moe_block_skinny_amd import binding as mb
from moe_block_skinny_amd import synth
from oracle import oracle as orc
from tests import inputs
from tests.gpu_util import dev, host, widen, say, fp32_sum_bound

pytestmark = pytest.mark.gpu

SHAPES = {"gemv": [1, 2], "splitk": [1, 3, 8], "mfma": [1, 9, 33, 64], "auto": [1, 2, 5, 8, 16, 64]}


@contextlib.contextmanager
def variant(name):
    prev = mb.set_variant(name)
    try:
        yield
    finally:
        mb.set_variant(prev)


def run(Xh, Wrh, Wlh, k, bias=None, bias_ld=0, latent_dtype=torch.float32):
    B, d = Xh.shape
    E, L = Wrh.shape[0], Wlh.shape[0]
    ids = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((B, k), float("nan"), device="cuda")
    plan = torch.full((mb.plan_words(B, k, E),), -7, dtype=torch.int32, device="cuda")
    lat = torch.full((B, L), float("nan"), dtype=latent_dtype, device="cuda")
    lo = torch.full((B, E), float("nan"), device="cuda")
    dt = mb.DT_BF16 if Xh.dtype == np.uint16 else mb.DT_F32
    ws = mb.workspace(mb.workspace_bytes(mb.OP_ROUTE_LATENT, dt, B=B, d=d, E=E, k=k, N=L))
    mb.moe_route_latent(dev(Xh), dev(Wrh), dev(Wlh), k, ids, w, plan, lat, ws,
                        bias=None if bias is None else dev(bias), bias_ld=bias_ld, logits_out=lo)
    torch.cuda.synchronize()
    return host(ids), host(w), host(plan), host(lat), host(lo)


def ints(a):
    return synth.to_bf16_bits(np.asarray(a, np.float32))


@pytest.mark.parametrize("var", ["auto", "gemv", "splitk", "mfma"])
def test_route_latent_integer_exact(var):
    rng = np.random.default_rng(41)
    E, d, k, L = 384, 7168, 8, 1024
    Wri = rng.integers(-1, 2, (E, d)) * (rng.random((E, d)) < 0.01)
    Wli = rng.integers(-3, 4, (L, d))
    Wr, Wl = ints(Wri), ints(Wli)
    for B in SHAPES[var]:
        say("route_latent integer", var, "B", B)
        Xi = rng.integers(-2, 3, (B, d))
        Xh = ints(Xi)
        Lg, ids, w, pl = orc.route(Xh, Wr, k)
        with variant(var):
            g_ids, g_w, g_pl, g_lat, g_l = run(Xh, Wr, Wl, k)
        assert np.array_equal(g_l, Lg), (var, B)
        assert np.array_equal(g_lat, orc.latent_projection(Xh, Wl)), (var, B)
        assert np.array_equal(g_lat, (Xi @ Wli.T).astype(np.float64)), (var, B)
        assert np.array_equal(g_ids, ids) and np.array_equal(g_pl, pl), (var, B)
        assert np.max(np.abs(g_w - w)) <= 1e-6
        if var != "auto":
            assert var in mb.last_variant()


@pytest.mark.parametrize("name", ["tp16_b1", "tp16_b8", "tp8_b64"])
def test_route_latent_workloads(name):
    c = inputs.case(name)
    Wl = synth.latent_w(c.cfg, 0)
    ref = orc.latent_projection(c.X, Wl)
    bound = fp32_sum_bound(widen(c.X), widen(Wl))
    lbound = fp32_sum_bound(widen(c.X), widen(c.Wr)) + 2.0 ** -23 * np.abs(c.logits)
    for var in ["auto"] + (["gemv"] if c.cfg.B <= 2 else []) + ["mfma"]:
        for ldt in (torch.float32, torch.bfloat16):
            say("route_latent workload", name, var, ldt)
            with variant(var):
                g_ids, g_w, g_pl, g_lat, g_l = run(c.X, c.Wr, Wl, c.cfg.k, c.bias, c.bias_ld, ldt)
            assert np.array_equal(g_ids, c.ids) and np.array_equal(g_pl, c.plan), var
            assert np.max(np.abs(g_w - c.w)) <= 1e-5, var
            assert np.all(np.abs(g_l - c.logits) <= lbound), var
            extra = 0.0 if ldt == torch.float32 else 2.0 ** -8 * np.abs(ref)
            assert np.all(np.abs(g_lat - ref) <= bound + extra), (var, ldt)


@pytest.mark.parametrize("B,d,E,k,L", [(3, 1056, 20, 4, 16), (12, 2080, 36, 5, 48), (64, 1024, 512, 16, 8192)])
def test_route_latent_ragged(B, d, E, k, L):
    rng = np.random.default_rng(B + L)
    Xi = rng.integers(-2, 3, (B, d))
    Wri = rng.integers(-1, 2, (E, d)) * (rng.random((E, d)) < 0.05)
    Wli = rng.integers(-2, 3, (L, d))
    Xh, Wr, Wl = ints(Xi), ints(Wri), ints(Wli)
    Lg, ids, w, pl = orc.route(Xh, Wr, k)
    say("route_latent ragged B", B, "d", d, "E", E, "L", L)
    g_ids, g_w, g_pl, g_lat, g_l = run(Xh, Wr, Wl, k)
    assert np.array_equal(g_l, Lg)
    assert np.array_equal(g_lat, (Xi @ Wli.T).astype(np.float64))
    assert np.array_equal(g_ids, ids) and np.array_equal(g_pl, pl)
