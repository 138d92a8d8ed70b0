"""The one-launch block schedule (fused kernel) against the three-launch
schedule and the CPU oracle (needs an MI355X).

Both schedules run the same device functions with the same split of every
sum, so their outputs, ids and weights must agree bit for bit; both must
meet the oracle bars of the block (ids exact, weights 1e-5; for bf16 the
bars of check_block_output: per element |bf16(ref) - ref| + 2e-3 rms, and
max|err| <= 2e-2 rms where rounding leaves room for it).  Ragged shapes: d not a multiple of the
rows per workgroup, E not a multiple of the router's 4-row tasks, I and Is
giving an odd number of 2-pair tasks, B*k = 64 with fewer experts than
slots.
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

RAGGED = {
    "ragged_b3": synth.MoEConfig("ragged_b3", 3, 2080, 130, 6, 96, 64, "bf16", "gumbel"),
    "slots64_e20": synth.MoEConfig("slots64_e20", 4, 1024, 20, 16, 32, 32, "bf16", "plain"),
    "f32_b2": synth.MoEConfig("f32_b2", 2, 1024, 40, 4, 64, 32, "f32", "gumbel"),
    "noshared_b5": synth.MoEConfig("noshared_b5", 5, 3072, 64, 4, 128, 0, "bf16", "plain"),
}

_cases = {}


def case(name):
    if name not in _cases:
        _cases.clear()
        if name in RAGGED:
            c = inputs.Case(RAGGED[name], seed=3)
        else:
            c = inputs.case(name)
        cfg = c.cfg
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        W13 = torch.full((cfg.E, 2 * cfg.I, cfg.d), float("nan"), dtype=tdt, device="cuda")
        W2 = torch.full((cfg.E, cfg.d, cfg.I), float("nan"), dtype=tdt, device="cuda")
        for e in c.touched:
            W13[e] = dev(c.W13[e])
            W2[e] = dev(c.W2[e])
        Ws13 = None if c.Ws13 is None else dev(c.Ws13)
        Ws2 = None if c.Ws2 is None else dev(c.Ws2)
        _cases[name] = (c, (W13, W2, Ws13, Ws2))
    return _cases[name]


@contextlib.contextmanager
def schedule(name):
    prev = mb.set_block_schedule(name)
    try:
        yield
    finally:
        mb.set_block_schedule(prev)


def run(c, weights, ws=None, calls=1):
    cfg = c.cfg
    W13, W2, Ws13, Ws2 = weights
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dt = mb.DT_BF16 if cfg.dtype == "bf16" else mb.DT_F32
    if ws is None:
        ws = mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, dt, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k, I=cfg.I, Is=cfg.Is))
    bias = None if c.bias is None else dev(c.bias)
    X, Wr = dev(c.X), dev(c.Wr)
    outs = []
    for _ in range(calls):
        out = torch.full((cfg.B, cfg.d), float("nan"), dtype=tdt, device="cuda")
        ids = torch.full((cfg.B, cfg.k), -1, dtype=torch.int32, device="cuda")
        w = torch.full((cfg.B, cfg.k), float("nan"), device="cuda")
        mb.moe_block(X, Wr, cfg.k, W13, W2, out, ws, Ws13, Ws2, bias, c.bias_ld, ids, w)
        outs.append((out, ids, w))
        torch.cuda.synchronize()
        # no grid barrier of the fused schedule gave up waiting
        assert mb.workspace_status(ws) == 0
    return outs


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name", ["tp16_b1", "tp16_b8"] + list(RAGGED))
def test_fused_equals_launches_and_oracle(name):
    c, weights = case(name)
    cfg = c.cfg
    say("fused block", name, "B", cfg.B, "d", cfg.d, "E", cfg.E, "k", cfg.k, "I", cfg.I, "Is", cfg.Is)
    with schedule("fused"):
        (of, idf, wf), = run(c, weights)
        assert "fused" in mb.last_variant()
    with schedule("launches"):
        (ol, idl, wl), = run(c, weights)
        assert "fused" not in mb.last_variant()
    assert torch.equal(idf, idl)
    assert torch.equal(bits(wf), bits(wl))
    assert torch.equal(bits(of), bits(ol))
    ref = c.oracle_block()
    g = host(of)
    assert np.array_equal(host(idf), c.ids)
    assert np.max(np.abs(host(wf) - c.w)) <= 1e-5
    if cfg.dtype == "bf16":
        r_err, r_rnd = check_block_output(g, ref["out"])
        say("  max|err|/rms(out) %.5f, exact result rounded to bf16: %.5f" % (r_err, r_rnd))
    else:
        scale = rms(ref["out"])
        err = np.abs(g - ref["out"])
        say("  max|err|/rms(out)", err.max() / scale)
        assert err.max() <= 1e-4 * scale


@pytest.mark.parametrize("name", ["tp16_b8", "ragged_b3"])
def test_fused_back_to_back_calls(name):
    """Calls queued back to back on one workspace: each leaves the barrier
    words ready for the next, so all give the same bits."""
    c, weights = case(name)
    with schedule("fused"):
        outs = run(c, weights, calls=6)
    for out, ids, w in outs[1:]:
        assert torch.equal(bits(out), bits(outs[0][0]))
        assert torch.equal(ids, outs[0][1])
        assert torch.equal(bits(w), bits(outs[0][2]))


def test_fused_out_of_scope_is_refused():
    """B*k above 64 slots: the fused schedule reports MOE_EUNSUPPORTED rather
    than switching path silently."""
    c, weights = case("tp16_b8")
    cfg = c.cfg.with_batch(9)
    sub = inputs.Case(cfg, seed=0)
    W13, W2, Ws13, Ws2 = weights
    with schedule("fused"):
        with pytest.raises(mb.MoeError) as ei:
            run(sub, (W13, W2, Ws13, Ws2))
    assert ei.value.status == mb.EUNSUPPORTED
