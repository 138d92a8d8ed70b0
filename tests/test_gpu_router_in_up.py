"""The two-launch block schedule (router rows inside the gate/up launch, B <= 2)
against the three-launch schedule and the CPU oracle (needs an MI355X).

The gate/up launch's router workgroups play the router launch's 16 waves, so
every logit, and with it every id, weight and output, must agree bit for bit
with the three launches; both meet the oracle bars of the block (ids exact,
weights 1e-5, outputs as check_block_output).  The logit keys live in the
workspace header and the down launch zeroes them: calls with different
inputs back to back on one workspace must each match their own three-launch
result (a key left over from the previous call would be taken for this
call's).  Shapes: an odd number of router rows (the last workgroup scores
one), a per-expert bias, fp32, no shared expert.
"""
import contextlib

import numpy as np
import pytest
import torch

from moe_block_skinny_amd import binding as mb
from moe_block_skinny_amd import synth
from tests import inputs
from tests.gpu_util import check_block_output, dev, host, rms, say

pytestmark = pytest.mark.gpu

CASES = {
    "odd_e_b1": synth.MoEConfig("odd_e_b1", 1, 2080, 131, 6, 96, 64, "bf16", "gumbel"),
    "zipf_b2": synth.MoEConfig("zipf_b2", 2, 3072, 96, 8, 64, 64, "bf16", "zipf"),
    "f32_b2": synth.MoEConfig("f32_b2", 2, 1024, 40, 4, 64, 32, "f32", "gumbel"),
    "noshared_b1": synth.MoEConfig("noshared_b1", 1, 1024, 64, 4, 128, 0, "bf16", "plain"),
}

_cases = {}


def case(name, seed=3):
    key = (name, seed)
    if key not in _cases:
        _cases.clear()
        c = inputs.Case(CASES[name], seed=seed) if name in CASES else inputs.case(name)
        cfg = c.cfg
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        W13 = torch.full((cfg.E, 2 * cfg.I, cfg.d), float("nan"), dtype=tdt, device="cuda")
        W2 = torch.full((cfg.E, cfg.d, cfg.I), float("nan"), dtype=tdt, device="cuda")
        for e in c.touched:
            W13[e] = dev(c.W13[e])
            W2[e] = dev(c.W2[e])
        Ws13 = None if c.Ws13 is None else dev(c.Ws13)
        Ws2 = None if c.Ws2 is None else dev(c.Ws2)
        _cases[key] = (c, (W13, W2, Ws13, Ws2))
    return _cases[key]


@contextlib.contextmanager
def schedule(name):
    prev = mb.set_block_schedule(name)
    try:
        yield
    finally:
        mb.set_block_schedule(prev)


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def block(c, weights, ws, X=None):
    cfg = c.cfg
    W13, W2, Ws13, Ws2 = weights
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    bias = None if c.bias is None else dev(c.bias)
    out = torch.full((cfg.B, cfg.d), float("nan"), dtype=tdt, device="cuda")
    ids = torch.full((cfg.B, cfg.k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((cfg.B, cfg.k), float("nan"), device="cuda")
    mb.moe_block(dev(c.X) if X is None else X, dev(c.Wr), cfg.k, W13, W2, out, ws, Ws13, Ws2, bias, c.bias_ld,
                 ids, w)
    return out, ids, w


def workspace(cfg):
    dt = mb.DT_BF16 if cfg.dtype == "bf16" else mb.DT_F32
    return mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, dt, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k, I=cfg.I, Is=cfg.Is))


@pytest.mark.parametrize("name", ["tp16_b1"] + list(CASES))
def test_router_in_up_equals_launches_and_oracle(name):
    c, weights = case(name)
    cfg = c.cfg
    say("router rows in the gate/up launch", name, "B", cfg.B, "d", cfg.d, "E", cfg.E, "k", cfg.k)
    ws = workspace(cfg)
    with schedule("router_in_up"):
        o2, i2, w2 = block(c, weights, ws)
        torch.cuda.synchronize()
        assert "rows in the gate/up launch" in mb.last_variant()
        assert mb.workspace_status(ws) == 0
    with schedule("launches"):
        o3, i3, w3 = block(c, weights, ws)
        torch.cuda.synchronize()
        assert "rows in the gate/up launch" not in mb.last_variant()
    assert torch.equal(i2, i3)
    assert torch.equal(bits(w2), bits(w3))
    assert torch.equal(bits(o2), bits(o3))
    ref = c.oracle_block()
    assert np.array_equal(host(i2), c.ids)
    assert np.max(np.abs(host(w2) - c.w)) <= 1e-5
    g = host(o2)
    if cfg.dtype == "bf16":
        r_err, r_rnd = check_block_output(g, ref["out"])
        say("  max|err|/rms(out) %.5f, exact result rounded to bf16: %.5f" % (r_err, r_rnd))
    else:
        err = np.abs(g - ref["out"])
        say("  max|err|/rms(out)", err.max() / rms(ref["out"]))
        assert err.max() <= 1e-4 * rms(ref["out"])


@pytest.mark.parametrize("name", ["tp16_b1", "zipf_b2"])
def test_router_in_up_back_to_back_inputs(name):
    """Two inputs alternated on one workspace, queued without a sync: every
    call matches the three-launch result of its own input."""
    c, weights = case(name)
    cfg = c.cfg
    g = torch.Generator(device="cuda").manual_seed(11)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    xs = [dev(c.X), torch.randn((cfg.B, cfg.d), generator=g, device="cuda").to(tdt)]
    ws = workspace(cfg)
    with schedule("launches"):
        refs = [block(c, weights, ws, X=x) for x in xs]
    torch.cuda.synchronize()
    assert not torch.equal(refs[0][1], refs[1][1]), "the two inputs should route differently"
    with schedule("router_in_up"):
        got = [block(c, weights, ws, X=xs[i % 2]) for i in range(6)]
    torch.cuda.synchronize()
    assert mb.workspace_status(ws) == 0
    for i, (o, ids, w) in enumerate(got):
        ro, rids, rw = refs[i % 2]
        assert torch.equal(ids, rids), i
        assert torch.equal(bits(w), bits(rw)), i
        assert torch.equal(bits(o), bits(ro)), i


def test_router_in_up_outside_its_scope_takes_three_launches():
    """B = 8 (above the two tokens the header's keys hold) and the shared
    expert placed in the router launch: three launches, same bits."""
    c, weights = case("tp16_b8")
    ws = workspace(c.cfg)
    with schedule("router_in_up"):
        o2, i2, _ = block(c, weights, ws)
        torch.cuda.synchronize()
        assert "rows in the gate/up launch" not in mb.last_variant()
    with schedule("launches"):
        o3, i3, _ = block(c, weights, ws)
    torch.cuda.synchronize()
    assert torch.equal(i2, i3) and torch.equal(bits(o2), bits(o3))
    c1, weights1 = case("tp16_b1")
    ws1 = workspace(c1.cfg)
    prev = mb.set_shared_schedule("router")
    try:
        with schedule("router_in_up"):
            block(c1, weights1, ws1)
            torch.cuda.synchronize()
            assert "rows in the gate/up launch" not in mb.last_variant()
    finally:
        mb.set_shared_schedule(prev)
