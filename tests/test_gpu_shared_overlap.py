"""Where the shared expert runs at small batch (needs an MI355X): its tiles
first in the gate/up launch (the default), its gate/up in the router launch
(one pass over x), or the whole shared expert on a second stream
(moe_block_streams) overlapping routing and the routed gate/up.  All three
compute the same products in the same order, so output, ids and weights are
bit-identical; each meets the oracle's bars.  Ragged cases: a shared expert
wider than the routed ones, an odd number of shared tiles, d not a multiple
of the down rows per workgroup."""
import contextlib

import numpy as np
import pytest
import torch

from moe_block_skinny_amd import binding as mb
from moe_block_skinny_amd import synth
from tests import inputs
from tests.gpu_util import check_block_output, dev, host, say
from tests.test_gpu_parity import gpu_weights

pytestmark = pytest.mark.gpu

RAGGED = {
    "wide_shared_b3": synth.MoEConfig("wide_shared_b3", 3, 2080, 130, 6, 96, 128, "bf16", "gumbel"),
    "shared96_b5": synth.MoEConfig("shared96_b5", 5, 1056, 40, 4, 64, 96, "bf16", "plain"),
}


@contextlib.contextmanager
def shared_schedule(name):
    prev = mb.set_shared_schedule(name)
    try:
        yield
    finally:
        mb.set_shared_schedule(prev)


def outs(cfg):
    return (torch.full((cfg.B, cfg.d), float("nan"), dtype=torch.bfloat16, device="cuda"),
            torch.full((cfg.B, cfg.k), -1, dtype=torch.int32, device="cuda"),
            torch.full((cfg.B, cfg.k), float("nan"), device="cuda"))


@pytest.mark.parametrize("name", ["tp16_b1", "tp16_b8"] + sorted(RAGGED))
def test_shared_placements_give_the_same_bits(name):
    c = inputs.case(name) if name in synth.CONFIGS else inputs.Case(RAGGED[name], seed=5)
    cfg = c.cfg
    W13, W2, Ws13, Ws2 = gpu_weights(c)
    bias = None if c.bias is None else dev(c.bias)
    X, Wr = dev(c.X), dev(c.Wr)
    ws = mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, mb.DT_BF16, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k,
                                         I=cfg.I, Is=cfg.Is))
    res = {}
    for place in ("up", "router"):
        o, i, w = outs(cfg)
        with shared_schedule(place):
            mb.moe_block(X, Wr, cfg.k, W13, W2, o, ws, Ws13, Ws2, bias, c.bias_ld, i, w)
        torch.cuda.synchronize()
        say("shared in", place, name, mb.last_variant())
        res[place] = (o, i, w)
    side = torch.cuda.Stream()
    fork, join = torch.cuda.Event(), torch.cuda.Event()
    o, i, w = outs(cfg)
    for rep in range(3):   # back to back on one workspace
        mb.moe_block_streams(X, Wr, cfg.k, W13, W2, o, ws, side, fork, join, Ws13, Ws2, bias, c.bias_ld, i, w)
    torch.cuda.synchronize()
    say("shared on a side stream", name, mb.last_variant())
    assert "side stream" in mb.last_variant()
    res["stream"] = (o, i, w)
    ref = res["up"]
    for place in ("router", "stream"):
        assert torch.equal(res[place][1], ref[1]), place
        assert torch.equal(res[place][2].view(torch.int32), ref[2].view(torch.int32)), place
        assert torch.equal(res[place][0].view(torch.int16), ref[0].view(torch.int16)), place
    assert np.array_equal(host(ref[1]), c.ids)
    assert np.max(np.abs(host(ref[2]) - c.w)) <= 1e-5
    r_err, _ = check_block_output(host(ref[0]), c.oracle_block()["out"])
    say("  max|err|/rms %.5f" % r_err)


def test_side_stream_outside_its_scope_is_refused():
    """Batch 64 (matrix shapes) or no shared expert: MOE_EUNSUPPORTED."""
    c = inputs.case("tp8_b64")
    cfg = c.cfg
    W13, W2, Ws13, Ws2 = gpu_weights(c)
    ws = mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, mb.DT_BF16, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k,
                                         I=cfg.I, Is=cfg.Is))
    o, i, w = outs(cfg)
    side = torch.cuda.Stream()
    with pytest.raises(mb.MoeError) as ei:
        mb.moe_block_streams(dev(c.X), dev(c.Wr), cfg.k, W13, W2, o, ws, side, torch.cuda.Event(),
                             torch.cuda.Event(), Ws13, Ws2, dev(c.bias), c.bias_ld, i, w)
    assert ei.value.status == mb.EUNSUPPORTED
