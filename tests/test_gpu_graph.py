"""The block captured in a HIP graph (needs an MI355X): every replay, with
plain launches of other inputs on the same workspace in between, gives the
bits of the plain launch.  The library records no memset node (counters are
left at zero by the kernels themselves), so replays after the first see the
workspace as the first did."""
import pytest
import torch

from moe_block_skinny_amd import binding as mb
from tests import inputs
from tests.gpu_util import dev, say
from tests.test_gpu_parity import gpu_weights

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tp16_b1", "tp16_b8", "tp8_b64"])
def test_block_graph_replays_match_plain_launches(name):
    c = inputs.case(name)
    cfg = c.cfg
    W13, W2, Ws13, Ws2 = gpu_weights(c)
    ws = mb.workspace(mb.workspace_bytes(mb.OP_BLOCK, mb.DT_BF16, B=cfg.B, d=cfg.d, E=cfg.E, k=cfg.k,
                                         I=cfg.I, Is=cfg.Is))
    bias = None if c.bias is None else dev(c.bias)
    X, Wr = dev(c.X), dev(c.Wr)
    Xo = torch.flip(X, dims=[0]).contiguous()   # other tokens for the plain launches in between
    out = torch.empty((cfg.B, cfg.d), dtype=torch.bfloat16, device="cuda")
    other = torch.empty_like(out)

    def block(x, o):
        mb.moe_block(x, Wr, cfg.k, W13, W2, o, ws, Ws13, Ws2, bias, c.bias_ld)

    block(X, out)
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        block(X, out)
    torch.cuda.synchronize()
    say("graph", name, mb.last_variant())
    for rep in range(4):
        out.fill_(0)
        g.replay()
        block(Xo, other)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
